// Chain verification by modified rejection sampling, batched over sequences.
//
// "Speculative Decoding in Production: From Draft Models to EAGLE-3 Dynamic Trees"
// (blog.llmgo.top), section I.1: alpha_k = min(1, p(x_k)/q(x_k)) (step 1), accept
// while r_k <= alpha_k and stop at the first rejection (step 2), on rejection draw
// from max(0, p - q) normalised (step 3).  Readings where the page is silent:
// p = softmax(target / T), q = softmax(draft / T); a bonus token is drawn from the
// target row after the last accepted draft; draws are inverse-CDF in vocabulary
// order (smallest index whose inclusive prefix reaches u * total).
//
// Two kernels (three with packed output), ordered by the stream:
//
//  chain_stats  grid = B x R x C: R = K+1 target rows (+ K draft rows when draft logits
//               are given), C chunks per row.  Each wave of a workgroup reduces one
//               contiguous quarter of a chunk (non-temporal 16-byte loads) to
//               (o, s) = (max(l) * log2(e)/T, sum exp2(l * log2(e)/T - o)), and the lane
//               holding the row's drafted token x_k copies l(x_k) out of its registers.
//               This is the pass that reads every logit, once.
//  chain_pool   grid = B x S/4 tasks (see chain_pool_kernel): every task of a sequence
//               combines the partials into per-row (O, S) and evaluates p(x_k), q(x_k),
//               alpha_k and the accept tests of all drafted positions at once (one lane
//               per position), taking the first rejection n with a wave ballot.  After a
//               rejection against draft rows, each task sums max(0, p - q) over its 4
//               segments of the row pair (a segment = one 16-byte vector per lane), and the
//               token is drawn from those masses.  A bonus or one-hot draw samples a target
//               row whose piece masses (one per wave partial) the stats pass already holds,
//               so one task per sequence reads only the piece that holds the draw.
//  chain_pack   grid = 1, only for packed output: offsets and packed tokens.
//
// Softmax is evaluated in the exp2 domain: with scale = log2(e)/T,
// p_i = exp2(l_i * scale - O) / S, where O is the float max(l) * scale used by every
// term and S = sum_chunks s_c * exp2(o_c - O).  Per-element work is fp32; cross-lane,
// cross-chunk and prefix sums are fp64.
#include <math.h>

#include <atomic>
#include <chrono>
#include <random>

#include "device_common.h"
#include "host_runtime.h"
#include "ngram_body.h"
#include "spec_verify.h"

namespace specv {

enum ChainMode : int {
  kModeInvalid = 0,
  kModeResidual = 1,
  kModeBonus = 2,
  kModeOneHot = 3,
  kModeFallbackP = 4,
  kModeGreedy = 5,  // temperature 0: the emitted row is complete after the decision
};

// Partial of one wave's share of a chunk.  Sampled rows: o = max(l) * scale (-inf if every
// logit is -inf) and s = sum exp2(l * scale - o).  Greedy rows (temperature 0): o = the
// largest logit and s = its smallest vocabulary index.
struct RowStat {
  float o;
  float pad;
  double s;
};

// Segment masses pass between the tasks of one pool launch through slots of two tagged
// 64-bit words (see the hand-over words in device_common.h), tagged with the call's
// generation number.  The generation mixes a number the host draws for each call (a
// process-wide counter with a random start) with a counter in the workspace that the
// stats kernel advances on every run, so that it changes even when a captured graph
// replays the same launch arguments; it is never 0.
struct SlotDouble {
  uint64_t lo, hi;
};

__device__ __forceinline__ void put_slot(SlotDouble* p, double v, uint32_t gen, bool local = false) {
  put_tagged_double(&p->lo, v, gen, local);
}

// Reads a slot; false if it has not been written during this call.
__device__ __forceinline__ bool get_slot(const SlotDouble* p, uint32_t gen, double* v) {
  return get_tagged_double(&p->lo, gen, v);
}

// 1 / s for a row sum s >= 1: the hardware reciprocal refined by one Newton step (its error
// squared, well below the fp32 rounding every use applies), instead of an IEEE division on
// the decision's critical path (measured: 0.1 us less pool time per call).
__device__ __forceinline__ double inv_row_sum(double s) {
  const double r = __builtin_amdgcn_rcp(s);
  return fma(r, fma(-s, r, 1.0), r);
}

struct ChainDecision {
  int mode;
  int n;         // accepted drafts
  int kb;        // draft length
  int excl_tok;  // one-hot mode: token removed from the residual
  int row;       // position whose row(s) the final draw samples
  float scale;   // log2(e) / T
  float Ot, Od;  // row offsets (target, draft)
  float invSt, invSd;
  float p_excl;  // one-hot mode: p_n(x_n)
  float uf;      // the final draw's uniform
  double St, Sd;
};

// A decision read from shared memory, held in scalar registers.
__device__ __forceinline__ ChainDecision uniform_decision(const ChainDecision& s) {
  ChainDecision d;
  d.mode = uniform(s.mode);
  d.n = uniform(s.n);
  d.kb = uniform(s.kb);
  d.excl_tok = uniform(s.excl_tok);
  d.row = uniform(s.row);
  d.scale = uniform(s.scale);
  d.Ot = uniform(s.Ot);
  d.Od = uniform(s.Od);
  d.invSt = uniform(s.invSt);
  d.invSd = uniform(s.invSd);
  d.p_excl = uniform(s.p_excl);
  d.uf = uniform(s.uf);
  d.St = uniform(s.St);
  d.Sd = uniform(s.Sd);
  return d;
}


struct ChainArgs {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* draft_len;
  const float* temperature;
  const float* u_accept;
  const float* u_final;
  int B, K, V, C, R;
  int nv;               // vectors per lane in one stats chunk (a chunk = nv segments)
  int S;                // pool segment slots per row: ceil(V / segment) rounded up to whole tasks
  int32_t* out_tokens;
  int32_t* out_num;
  float* out_probs;
  int32_t* out_packed;
  int32_t* out_offsets;
  uint32_t gen;         // the host's number for this call (see pool_generation)
  int poll_limit;       // polls of a missing hand-over word before the wait gives up
  uint32_t* runs;       // workspace counter advanced by every stats kernel run
  RowStat* part;        // [B, R, C, 4] partials, one per wave of each chunk
  float* gath;          // [B, R] logit of the drafted token in each scoring row
  SlotDouble* wseg;     // [B, S] slots: mass of the final draw's weights per segment
  ChainDecision* decs;  // [B] decisions of chain_decide_kernel for the pool kernel
  int decided;          // the pool reads its decisions from decs (else it decides itself)
  int xcd_local;        // fused launch: each sequence's workgroups share an XCD, hand-overs stay in its L2
  int stats_copy;              // the stats pass copies the drafted tokens' logits out (else the lookup does)
  // single-launch path (see chain_single_kernel): hand-over words tagged with seq_tag
  uint32_t* epoch;             // [B] per-sequence run counters
  uint64_t* tpart;             // [B, tstride] partials ([R, C, kWaves] of 3 words): o, then s as a tagged double
  uint64_t* tprop;             // [B, 2K+1] lookup results: draft length, tokens [K], their logits [K]
  uint64_t* status;            // [B, sstride] one word per workgroup (see SeqStatus) or helper
  int tstride, sstride;        // words per sequence in tpart and status
  SlotDouble* tmass;           // [B, K, S] slots: residual mass of each segment, should position k reject
  uint64_t* tdec;              // [B, kFusedDecisionWords] the fused path's decisions
  unsigned long long* stamps;  // phase timestamps (measurement only; see spec_chain_phase_stamps), or null
  size_t stamps_pool;          // index of the pool tasks' first stamp
};

// Phase timestamps (the device's constant 100 MHz clock), written by thread 0 when the
// caller asked for them.  Stats workgroup g: stamps[2g] start, [2g+1] end.  Pool task t
// (t = b * CP + c for task c of sequence b): stamps[stamps_pool + kStampsPerTask * t + i] for
// the phases of kPoolPhase, the last word holding (b << 32) | (c << 8) | mode.
constexpr int kStampsPerTask = 6;
enum PoolPhase : int { kPhStart = 0, kPhDecided = 1, kPhPublished = 2, kPhGathered = 3, kPhEnd = 4, kPhInfo = 5 };
// Phases of a single-launch workgroup (stamps[kStampsPerTask * w + i] for workgroup w of the
// sequences' workgroups, in grid order after the lookup's).
enum SinglePhase : int { kSgStart = 0, kSgPublished = 1, kSgGathered = 2, kSgDecided = 3, kSgDrawn = 4, kSgEnd = 5 };
// Phases of a fused launch (G stats workgroups, B finishers, B x CP helpers): stats chunk g
// (sequence, row, chunk order) at stamps[2g] (start) and [2g+1] (partials published); the
// finisher of sequence b at stamps[2G + kFinisherStamps * b + i]; helper h = b * CP + c at
// stamps[2G + kFinisherStamps * B + kHelperStamps * h + i].
constexpr int kFinisherStamps = 4;
constexpr int kHelperStamps = 7;
enum FinisherPhase : int { kFnGathered = 0, kFnDecided = 1, kFnEnd = 2, kFnMode = 3 };
enum HelperPhase : int {
  kHpStart = 0, kHpSeen = 1, kHpPublished = 2, kHpLocated = 3, kHpNarrowed = 4, kHpExit = 5, kHpInfo = 6
};

// A stamp base from kNoStamp on writes nothing (callers whose layout has no word for a helper's
// phase pass it).
constexpr size_t kNoStamp = ~size_t{0} >> 1;

__device__ __forceinline__ void stamp(const ChainArgs& a, size_t i) {
  if (a.stamps && i < kNoStamp && threadIdx.x == 0) a.stamps[i] = __builtin_amdgcn_s_memrealtime();
}

// Generation of the slot words of this pool launch (see SlotDouble): the host's number
// mixed with the workspace counter as the stats kernel of this call left it.
__device__ __forceinline__ uint32_t pool_generation(const ChainArgs& a) {
  const uint32_t g = a.gen ^ (load_agent(a.runs) * 0x9e3779b1u);
  return g != 0u ? g : 0x2545f491u;
}

// Tag of sequence b's hand-over words on the single-launch path: the host's number for the call
// mixed with the sequence's run counter, which its last pool task advances once every
// workgroup of the sequence has read it (so that a captured graph replaying the same launch
// arguments still gets new tags; kernels of a stream run one after another, so no word of a
// run is written during the next), and with the address of the launch's dispatch packet in
// the queue: after a wait gave up, workgroups of the run that start late may read the advanced
// counter, and the packet address keeps their words apart from those of the next launch.
// (seq_tag_from: the same from a counter value read beforehand, so that the read can go out
// with a workgroup's streaming loads and be used once they are consumed.)
__device__ __forceinline__ uint32_t seq_tag_from(const ChainArgs& a, uint32_t run) {
  const uint64_t packet = reinterpret_cast<uint64_t>(__builtin_amdgcn_dispatch_ptr()) >> 6;  // 64-byte packets
  const uint32_t g = a.gen ^ (static_cast<uint32_t>(packet) * 0x85ebca6bu) ^ (run * 0x9e3779b1u);
  return g != 0u ? g : 0x2545f491u;
}

__device__ __forceinline__ uint32_t seq_tag(const ChainArgs& a, int b) { return seq_tag_from(a, load_agent(a.epoch + b)); }

template <int DT>
__device__ __forceinline__ const void* target_row(const ChainArgs& a, int b, int k) {
  return static_cast<const char*>(a.target) +
         (static_cast<size_t>(b) * (a.K + 1) + k) * static_cast<size_t>(a.V) * Elem<DT>::kBytes;
}

template <int DT>
__device__ __forceinline__ const void* draft_row(const ChainArgs& a, int b, int k) {
  return static_cast<const char*>(a.draft) +
         (static_cast<size_t>(b) * a.K + k) * static_cast<size_t>(a.V) * Elem<DT>::kBytes;
}

// An element of a caller's input array.  SCALAR: read through the scalar cache, for an array
// that no workgroup of the launch writes (not the draft lengths and tokens of a launch whose
// lookup writes them): with a workgroup-uniform index it is one scalar load, which the
// sequence's first workgroup brings into the cache for the rest, and which does not queue
// behind the streaming vector loads in flight on its compute unit.  The fused launch's stats
// workgroups read their sequence's length and temperature so before their chunk's loads can
// go out (measured at B=64, K=5, V=128256 bf16: greedy calls 27.5 -> 26.4 us, sampled calls
// unchanged); the separate stats pass and the single launch keep vector loads, which measured
// faster there (B=256, K=8, V=152064: 185.8 against 190.7 us for the pass; B=1, K=5,
// V=32000 fp32: 9.2 against 9.6 us per call).
template <bool SCALAR = false, class T>
__device__ __forceinline__ T input_load(const T* p, size_t i) {
  if (!SCALAR) return p[i];
  using CT = const __attribute__((address_space(4))) T;
  return reinterpret_cast<CT*>(reinterpret_cast<uintptr_t>(p))[i];
}

// Draft length of sequence b clamped to [0, K] (an out-of-range value is flagged later).
template <bool SCALAR = false>
__device__ __forceinline__ int clamped_len(const ChainArgs& a, int b) {
  if (!a.draft_len) return a.K;
  const int v = input_load<SCALAR>(a.draft_len, b);
  return v < 0 ? 0 : (v > a.K ? a.K : v);
}

// Temperature 0 selects greedy verification for a sequence.
template <bool SCALAR = false>
__device__ __forceinline__ bool is_greedy(const ChainArgs& a, int b) {
  return input_load<SCALAR>(a.temperature, b) == 0.f;
}

// Row rr of the stats grid: rr <= K is target row rr, otherwise draft row rr-K-1
// (draft rows exist only when draft logits are given; then R = 2K+1, else R = K+1; a
// greedy sequence reads no draft row).
__device__ __forceinline__ bool row_needed(const ChainArgs& a, int rr, int kb, bool greedy) {
  return rr <= a.K ? (rr <= kb) : (!greedy && a.draft != nullptr && rr - (a.K + 1) < kb);
}

// Drafted position whose token row rr scores (target row k or draft row k, k < kb), else -1.
__device__ __forceinline__ int row_position(const ChainArgs& a, int rr, int kb) {
  const int k = rr <= a.K ? rr : rr - (a.K + 1);
  return k < kb ? k : -1;
}

// ---------------------------------------------------------------- decision


// A sequence's inputs to the decision: its chunk partials ([R][C * kWaves]), drafted tokens
// ([K]), copied logits of the drafted tokens ([R], target row k at k, draft row k at K+1+k),
// accept-test uniforms ([K]), temperature, final uniform and raw draft length -- in the
// workspace and the caller's arrays, or staged in shared memory by a workgroup of the
// single-launch path.
struct SeqInputs {
  const RowStat* part;
  const int32_t* tokens;
  const float* gath;
  const float* u_accept;
  float T, uf;
  int kb_raw;
};

__device__ __forceinline__ SeqInputs seq_inputs(const ChainArgs& a, int b) {
  return SeqInputs{a.part + static_cast<size_t>(b) * a.R * a.C * kWaves,
                   a.tokens + static_cast<size_t>(b) * a.K,
                   a.gath + static_cast<size_t>(b) * a.R,
                   a.u_accept + static_cast<size_t>(b) * a.K,
                   input_load(a.temperature, b),
                   input_load(a.u_final, b),
                   a.draft_len ? input_load(a.draft_len, b) : a.K};
}

// No work between the decision's combining of the partials and the decision itself.
struct NoMidStep {
  __device__ void operator()(const float*, const double*) const {}
};

// Called by every lane of every pool task of sequence b: combines the sequence's chunk
// partials, decides and leaves the decision in *out (shared memory) -- identically in
// every task: same data, same arithmetic, same order.  With write_outputs it also writes
// the count and the probabilities (and a -1 row for invalid input).  The loads of a batch
// of rows are all issued before any is used.  kb = the draft length clamped to [0, K].
// mid(sO, sS), called by every lane once the rows' offsets and sums are in shared memory
// (sampled sequences: sO[r], sS[r] of row r as indexed by the partials), may use them before
// the decision is taken.
template <int DT, class Mid = NoMidStep>
__device__ __forceinline__ void chain_decide(const ChainArgs& a, int b, int kb, const SeqInputs& in,
                                             bool write_outputs, ChainDecision* out, Mid mid = Mid()) {
  __shared__ float sO[2 * SPEC_MAX_K + 1];
  __shared__ double sS[2 * SPEC_MAX_K + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int R = a.R, C = a.C * kWaves;  // C = partials per row (one per wave of a chunk)

  // Wave 0, lane k: the inputs of drafted position k.
  const int k = lane;
  const bool active = w == 0 && k < kb;
  int x = 0;
  float u = 1.f, gt = 0.f, gd = 0.f;
  if (active) {
    x = in.tokens[k];
    u = in.u_accept[k];
    gt = in.gath[k];
    if (a.draft) gd = in.gath[a.K + 1 + k];
  }
  const float T = in.T;
  const float uf = in.uf;
  const int kb_raw = in.kb_raw;
  const bool greedy = T == 0.f;

  // Per-row (O, S) from the partials -- for a greedy sequence the row argmax instead:
  // each 16-lane group of the workgroup combines one row of logits (16 rows at a time), lane
  // r taking partials r, r+16, ... straight from memory (the first kRegPer of them in
  // registers, all loads issued before any is used); the group's lane 15 leaves the row's
  // result in shared memory.
  __shared__ int sA[2 * SPEC_MAX_K + 1];  // greedy: argmax of each target row
  const int grp = tid >> 4;  // 16-lane group
  const int r = tid & 15;
  const int row_lane15 = (lane & ~15) | 15;
  constexpr int kRegPer = 4;
  for (int r0 = 0; r0 < R; r0 += kThreads / 16) {
    const int rr = r0 + grp;
    const bool live = rr < R && row_needed(a, rr, kb, greedy);
    const RowStat* ps = in.part + static_cast<size_t>(live ? rr : 0) * C;
    RowStat st[kRegPer];
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) {
      const int c = r + 16 * j;
      st[j] = live && c < C ? ps[c] : RowStat{-INFINITY, 0.f, static_cast<double>(INT_MAX)};
    }
    if (greedy) {
      float v = -INFINITY;
      int idx = INT_MAX;
      for (int j = 0; j < kRegPer; ++j) {
        const int ci = static_cast<int>(st[j].s);
        if (better(st[j].o, ci, v, idx)) {
          v = st[j].o;
          idx = ci;
        }
      }
      for (int c = r + 16 * kRegPer; live && c < C; c += 16) {
        const RowStat s2 = ps[c];
        const int ci = static_cast<int>(s2.s);
        if (better(s2.o, ci, v, idx)) {
          v = s2.o;
          idx = ci;
        }
      }
      row16_argmax(v, idx);
      if (live && r == 15) sA[rr] = idx;
    } else {
      float om = -INFINITY;
#pragma unroll
      for (int j = 0; j < kRegPer; ++j) om = fmaxf(om, st[j].o);
      for (int c = r + 16 * kRegPer; live && c < C; c += 16) om = fmaxf(om, ps[c].o);
      om = __shfl(row16_inclusive_max(om), row_lane15);
      double sum = 0.0;
#pragma unroll
      for (int j = 0; j < kRegPer; ++j)
        if (st[j].o != -INFINITY) sum += st[j].s * static_cast<double>(exp2_fast(st[j].o - om));
      for (int c = r + 16 * kRegPer; live && c < C; c += 16) {
        const RowStat s2 = ps[c];
        if (s2.o != -INFINITY) sum += s2.s * static_cast<double>(exp2_fast(s2.o - om));
      }
      sum = row16_inclusive_sum(sum);
      if (live && r == 15) {
        sO[rr] = om;
        sS[rr] = sum;
      }
    }
  }
  __syncthreads();
  mid(sO, sS);

  if (w == 0 && greedy) {
    // One lane per drafted position: accepted iff the draft is its target row's argmax;
    // the emitted row ends with the argmax of the row after the last accepted draft.
    bool bad = false, accepted = true;
    if (active) {
      bad = x < 0 || x >= a.V;
      accepted = x == sA[k];
    }
    const unsigned long long rej = __ballot(active && !accepted);
    const unsigned long long badm = __ballot(active && bad);
    const int n = rej ? (__ffsll(static_cast<long long>(rej)) - 1) : kb;
    const bool invalid = badm != 0ull || kb_raw < 0 || kb_raw > a.K;
    if (write_outputs) {
      if (a.out_probs && k < a.K) {  // p, q and alpha are not defined at temperature 0
        float* pr = a.out_probs + (static_cast<size_t>(b) * a.K + k) * 3;
        pr[0] = pr[1] = pr[2] = 0.f;
      }
      int32_t* ot = a.out_tokens + static_cast<size_t>(b) * (a.K + 1);
      for (int kk = lane; kk <= a.K; kk += 64) ot[kk] = invalid ? -1 : (kk < n ? x : (kk == n ? sA[n] : -1));
      if (lane == 0) a.out_num[b] = invalid ? -1 : n;
    }
    if (lane == 0) {
      ChainDecision d{};
      d.mode = invalid ? kModeInvalid : kModeGreedy;
      d.n = n;
      d.kb = kb;
      *out = d;
    }
  }
  if (w == 0 && !greedy) {
    // One lane per drafted position: p(x_k), q(x_k), alpha_k and the accept test.
    const float scale = kLog2e / T;
    bool bad = false, accepted = true;
    float P = 0.f, Q = 0.f, alpha = 0.f;
    if (active) {
      if (x < 0 || x >= a.V || !(u > 0.f && u <= 1.f)) {
        bad = true;
      } else {
        P = static_cast<float>(static_cast<double>(exp2_fast(fmaf(gt, scale, -sO[k]))) * inv_row_sum(sS[k]));
        if (a.draft) {
          const int rd = a.K + 1 + k;
          Q = static_cast<float>(static_cast<double>(exp2_fast(fmaf(gd, scale, -sO[rd]))) * inv_row_sum(sS[rd]));
        } else {
          Q = 1.f;
        }
        alpha = Q > 0.f ? fminf(1.f, P / Q) : (P > 0.f ? 1.f : 0.f);
        accepted = u <= alpha;
      }
    }
    const unsigned long long rej = __ballot(active && !accepted);
    const unsigned long long badm = __ballot(active && bad);
    const int n = rej ? (__ffsll(static_cast<long long>(rej)) - 1) : kb;
    const bool invalid = badm != 0ull || !(T > 0.f) || !(T <= 3.4e38f) || kb_raw < 0 || kb_raw > a.K ||
                         !(uf > 0.f && uf <= 1.f);
    const float Pn = lane_broadcast(P, n < 64 ? n : 0);
    const int xn = lane_broadcast(x, n < 64 ? n : 0);
    if (write_outputs) {
      if (a.out_probs && k < a.K) {
        float* pr = a.out_probs + (static_cast<size_t>(b) * a.K + k) * 3;
        const bool keep = active && !invalid;
        pr[0] = keep ? P : 0.f;
        pr[1] = keep ? Q : 0.f;
        pr[2] = keep ? alpha : 0.f;
      }
      if (invalid) {  // a valid sequence's row is written by its final draw
        int32_t* ot = a.out_tokens + static_cast<size_t>(b) * (a.K + 1);
        for (int kk = lane; kk <= a.K; kk += 64) ot[kk] = -1;
      }
      if (lane == 0) a.out_num[b] = invalid ? -1 : n;
    }
    if (lane == 0) {
      ChainDecision d{};
      d.n = n;
      d.kb = kb;
      d.scale = scale;
      d.uf = uf;
      d.excl_tok = -1;
      if (invalid) {
        d.mode = kModeInvalid;
      } else if (n == kb) {
        d.mode = kModeBonus;
        d.row = kb;
      } else if (a.draft) {
        d.mode = kModeResidual;
        d.row = n;
        d.Od = sO[a.K + 1 + n];
        d.Sd = sS[a.K + 1 + n];
        d.invSd = static_cast<float>(inv_row_sum(d.Sd));
      } else {
        d.mode = kModeOneHot;
        d.row = n;
        d.excl_tok = xn;
        d.p_excl = Pn;
      }
      if (!invalid) {
        d.Ot = sO[d.row];
        d.St = sS[d.row];
        d.invSt = static_cast<float>(inv_row_sum(d.St));
      }
      *out = d;
    }
  }
  __syncthreads();
}

// A wave's (largest logit, smallest index) over its share of chunk c (raw as load_wave_span
// leaves it).  The lane visits its elements in increasing vocabulary order, so a strict '>'
// keeps the first maximum; elements past V read as -inf and never replace the lane's first one.
template <int DT, int NV, bool VEC>
__device__ __forceinline__ void wave_argmax_partial(u32x4 (&raw)[NV], int c, int V, float* v_out, int* idx_out) {
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr int kChunk = ChunkShape<DT, NV>::kChunk;
  constexpr int kSpan = kChunk / kWaves;  // elements of one wave's quarter
  const int wv = static_cast<int>(threadIdx.x >> 6);
  const int ln = static_cast<int>(threadIdx.x & 63);
  const int first = c * kChunk + wv * kSpan + ln * E;
  float v = -INFINITY;
  int idx = first < V ? first : INT_MAX;
  // With vector loads, the packed registers count as rewritten here, so that no unpacked
  // element is shared with (and kept alive for) the sampling path.
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < NV; ++j) asm volatile("" : "+v"(raw[j]));
  }
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float l = EL::get(raw[j], i);
      if (l > v) {
        v = l;
        idx = c * kChunk + wv * kSpan + (j * 64 + ln) * E + i;
      }
    }
  wave_argmax(v, idx);
  *v_out = v;
  *idx_out = idx;
}

// A wave's softmax partial of its share of a chunk: o = its largest logit times `scale`
// (log2(e) / T, so that o is in the exp2 domain) and s = the sum of exp2(l * scale - o) over
// its elements, in fp64 across lanes; (-inf, 0) when every element is -inf.
template <int DT, int NV>
__device__ __forceinline__ void wave_softmax_partial(const u32x4 (&raw)[NV], float scale, float* o_out,
                                                     double* s_out) {
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  // The lane's vectors in parts of at most 4 (two parts for 8 vectors), each with its own
  // offset: a part's sums run while the later parts' loads are still in flight, and the
  // parts combine at the end (measured: 2-4 % less kernel time than one offset for all).
  constexpr int kParts = NV >= 16 ? 4 : (NV >= 2 ? 2 : 1);
  constexpr int kPer = NV / kParts;
  float o = -INFINITY, s = 0.f;
  float po[kParts], ps[kParts];
#pragma unroll
  for (int q = 0; q < kParts; ++q) {
    float m = -INFINITY;
#pragma unroll
    for (int j = q * kPer; j < (q + 1) * kPer; ++j)
#pragma unroll
      for (int i = 0; i < E; ++i) m = fmaxf(m, EL::get(raw[j], i));
    po[q] = -INFINITY;
    ps[q] = 0.f;
    if (m != -INFINITY) {
      const float oq = m * scale;
      float acc = 0.f, acc2 = 0.f;
#pragma unroll
      for (int j = q * kPer; j < (q + 1) * kPer; ++j)
#pragma unroll
        for (int i = 0; i < E; i += 2) {
          acc += exp2_fast(fmaf(EL::get(raw[j], i), scale, -oq));
          acc2 += exp2_fast(fmaf(EL::get(raw[j], i + 1), scale, -oq));
        }
      po[q] = oq;
      ps[q] = acc + acc2;
    }
    o = fmaxf(o, po[q]);
  }
  if (o != -INFINITY) {
#pragma unroll
    for (int q = 0; q < kParts; ++q)
      if (po[q] != -INFINITY) s += ps[q] * exp2_fast(po[q] - o);
  }
  const float ow = wave_max(o);
  const double contrib = (o == -INFINITY) ? 0.0 : static_cast<double>(s) * static_cast<double>(exp2_fast(o - ow));
  *o_out = ow;
  *s_out = wave_sum(contrib);
}

// One chunk g (in (sequence, row, chunk) order) of one row, reduced by one workgroup: each of
// its waves makes one partial of its quarter of the chunk (one contiguous span, see
// load_wave_span).  ALL_ROWS: every target row is read and no drafted logit is copied out (the
// draft lengths and tokens are being written by the same launch; see ngram_chain_stats_kernel).
// si: this workgroup's stamp pair.
template <int DT, int NV, bool VEC, bool ALL_ROWS>
__device__ __forceinline__ void chain_stats_body(const ChainArgs& a, int g, size_t si) {
  stamp(a, si);
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr int kChunk = ChunkShape<DT, NV>::kChunk;
  constexpr int kSpan = kChunk / kWaves;  // elements of one wave's quarter
  const int c = g % a.C;
  const int rr = (g / a.C) % a.R;
  const int b = g / (a.C * a.R);
  const int kb = ALL_ROWS ? a.K : clamped_len(a, b);
  const bool greedy = is_greedy(a, b);
  if (!row_needed(a, rr, kb, greedy)) {
    stamp(a, si + 1);
    return;
  }
  const void* row = rr <= a.K ? target_row<DT>(a, b, rr) : draft_row<DT>(a, b, rr - (a.K + 1));
  RowStat* out = a.part + ((static_cast<size_t>(b) * a.R + rr) * a.C + c) * kWaves + (threadIdx.x >> 6);

  u32x4 raw[NV];
  load_wave_span<DT, NV, VEC, true>(raw, row, a.V, c);
  const int wv = static_cast<int>(threadIdx.x >> 6);
  const int ln = static_cast<int>(threadIdx.x & 63);

  if (greedy) {  // (largest logit, smallest index) of the wave's share
    float v;
    int idx;
    wave_argmax_partial<DT, NV, VEC>(raw, c, a.V, &v, &idx);
    if (ln == 0) *out = RowStat{v, 0.f, static_cast<double>(idx)};
    stamp(a, si + 1);
    return;
  }
  const float scale = kLog2e / input_load(a.temperature, b);
  // (a run-time test rather than ALL_ROWS: with the copy compiled out, the compiler schedules the
  // pass with 74 instead of 63 VGPRs, 6 instead of 8 waves per SIMD)
  const int pos = a.stats_copy ? row_position(a, rr, kb) : -1;
  const int x = pos >= 0 ? a.tokens[static_cast<size_t>(b) * a.K + pos] : -1;

  // The lane holding the drafted token's logit copies it out (bit-exact).
  if (x >= 0 && x < a.V && x / kChunk == c) {
    const int local = x - c * kChunk;
    if (wv == local / kSpan && ln == (local / E) % 64) {
      const int j = (local % kSpan) / (64 * E);
      u32x4 v = raw[0];
#pragma unroll
      for (int jj = 1; jj < NV; ++jj)
        if (jj == j) v = raw[jj];
      a.gath[static_cast<size_t>(b) * a.R + rr] = EL::get(v, local % E);
    }
  }

  float ow;
  double sw;
  wave_softmax_partial<DT, NV>(raw, scale, &ow, &sw);
  // One partial per wave: no workgroup barrier in this kernel.
  if (ln == 0) *out = RowStat{ow, 0.f, sw};
  stamp(a, si + 1);
}

// grid = B x R x C: workgroup i reduces chunk g = xcd_blocked(i, G) of one row.
template <int DT, int NV, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_stats_kernel(ChainArgs a) {
  if (blockIdx.x == 0 && threadIdx.x == 0) __hip_atomic_fetch_add(a.runs, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  chain_stats_body<DT, NV, VEC, false>(a, xcd_blocked_index(), 2 * static_cast<size_t>(blockIdx.x));
}

// Where the prompt n-gram lookup drafts: the lookup of ngram_body.h and the row statistics of
// every target row run in one launch.  grid = B + B x (K+1) x C: workgroup i < B proposes for
// sequence i (draft tokens, lengths and matched n into the chain call's tokens, draft lengths
// and `match_n`) and copies the drafted tokens' logits out of their target rows (a token that
// is no vocabulary index is left for the decision to flag); the others reduce chunks as
// chain_stats_kernel does, over all K+1 target rows, since the draft lengths are not known when
// they start.
struct NgramArgs {
  const int32_t* context;
  const int32_t* context_len;
  int L_max, n_min, n_max;
  int32_t* match_n;
};

template <int DT, int NV, bool VEC>
__global__ __launch_bounds__(kThreads) void ngram_chain_stats_kernel(ChainArgs a, NgramArgs ng) {
  const int i = static_cast<int>(blockIdx.x);
  if (i < a.B) {
    if (i == 0 && threadIdx.x == 0) __hip_atomic_fetch_add(a.runs, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int32_t* tokens = const_cast<int32_t*>(a.tokens);
    const int len = ngram_propose_body<kThreads>(i, ng.context, ng.context_len, ng.L_max, ng.n_min, ng.n_max, a.K,
                                                 tokens, const_cast<int32_t*>(a.draft_len), ng.match_n);
    // lane k wrote token k of the draft above and reads it back
    for (int k = threadIdx.x; k < len; k += kThreads) {
      const int x = tokens[static_cast<size_t>(i) * a.K + k];
      if (x >= 0 && x < a.V) a.gath[static_cast<size_t>(i) * a.R + k] = Elem<DT>::value(target_row<DT>(a, i, k), x);
    }
    return;
  }
  const int G = static_cast<int>(gridDim.x) - a.B;
  chain_stats_body<DT, NV, VEC, true>(a, xcd_blocked(i - a.B, G), 0);
}

// ---------------------------------------------------------------- final draw

// Weight of one element in the final draw: max(0, p - q) after a rejection (residual),
// else p; zero for the excluded token (one-hot residual; excl = -1 excludes nothing).
// Logits past V read as -inf and weigh 0 in every mode.
__device__ __forceinline__ float draw_weight(bool residual, const ChainDecision& d, float lt, float ld, int e,
                                             int excl) {
  const float p = exp2_fast(fmaf(lt, d.scale, -d.Ot)) * d.invSt;
  float w = p;
  if (residual) w = fmaxf(0.f, p - exp2_fast(fmaf(ld, d.scale, -d.Od)) * d.invSd);
  return e == excl ? 0.f : w;
}

// Offsets and packed tokens of the whole batch (one workgroup, after the pass).
__device__ __forceinline__ void chain_pack(const ChainArgs& a) {
  __shared__ int s_i[kWaves];
  const int tid = threadIdx.x;
  const int per = (a.B + kThreads - 1) / kThreads;
  const int b0 = min(a.B, tid * per);
  const int b1 = min(a.B, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) {
    const int n = a.out_num[b];
    local += n >= 0 ? n + 1 : 0;
  }
  int total = 0;
  int run = block_exclusive_scan_int(local, s_i, &total);
  for (int b = b0; b < b1; ++b) {
    const int n = a.out_num[b];
    const int cnt = n >= 0 ? n + 1 : 0;
    a.out_offsets[b] = run;
    const int32_t* ot = a.out_tokens + static_cast<size_t>(b) * (a.K + 1);
    for (int i = 0; i < cnt; ++i) a.out_packed[run + i] = ot[i];
    run += cnt;
  }
  if (tid == 0) a.out_offsets[a.B] = total;
}

// Bonus and one-hot draws (and the fallback to p) sample target row d.row itself, minus the
// drafted token after a one-hot rejection, and write the emitted row.  The stats pass already
// summed that row in pieces: each wave partial (o, s) covers one contiguous quarter of a chunk,
// with mass s * exp2(o - O) / S (the same terms whose total is the row's S).  So the draw
// needs no pass over the whole row:
//  1. (direct_locate) wave 0 alone takes the units (pieces, or whole segments where a piece is
//     smaller than a segment), 64 per round, forms their masses from the partials, and scans
//     them in vocabulary order for the unit whose inclusive prefix reaches u * W (W = the
//     total);
//  2. (wave_segment_scan) each segment of that unit is held by one wave, lane l holding the
//     segment's vectors l, l + 64, l + 128, l + 192 (each load 1 KiB of contiguous memory):
//     the wave sums each vector's draw weights in fp32 and scans the sums in vocabulary order
//     in fp64, one round of 64 vectors at a time; the final prefix is the segment's mass;
//  3. (pick_segment, wave_segment_pick) the segment is picked from those masses, and the wave
//     holding it narrows from its registers to the vector, then the element.
// Unit masses come from the stats partials and segment masses from the draw weights, so the
// two agree to rounding; where u * W lies within that rounding of a boundary the last
// segment (or element) with mass is taken, as for every other draw.  With no mass left
// after removing the drafted token (all of the row on it), the draw falls back to p.

// Units of a direct draw on rows split into chunks of nv vectors a lane.
struct DirectUnits {
  int piece;  // elements of one wave partial
  int pper;   // pieces per unit
  int segs;   // segments per unit
  int unit;   // elements per unit
  int units;  // units in a row
};

template <int DT>
__device__ __forceinline__ DirectUnits direct_units(int nv, int V) {
  constexpr int kSeg = ChunkShape<DT, 1>::kSegment;
  DirectUnits u;
  u.piece = nv * (kSeg / kWaves);
  u.pper = nv >= kWaves ? 1 : kWaves / nv;
  u.segs = nv >= kWaves ? nv / kWaves : 1;
  u.unit = u.pper * u.piece;
  u.units = (V + u.unit - 1) / u.unit;  // <= S <= 4 * kThreads
  return u;
}

// Step 1, every lane calls it: wave 0 finds the unit holding u * W from the partials of row
// d.row (ps, C * kWaves of them) and the result is shared through shared memory.  *mode_io may
// turn from one-hot into the fallback to p.
template <int DT>
__device__ __forceinline__ void direct_locate(const ChainArgs& a, int b, const ChainDecision& d, int* mode_io,
                                              const RowStat* ps, int* usel_out, double* tunit_out) {
  __shared__ int s_unit, s_mode;
  __shared__ double s_tu;
  const int lane = threadIdx.x & 63;
  const DirectUnits U = direct_units<DT>(a.nv, a.V);
  const int nparts = a.C * kWaves;
  int mode = *mode_io;
  if ((threadIdx.x >> 6) == 0) {
    const int rounds = (U.units + 63) / 64;
    for (int attempt = 0; attempt < 2; ++attempt) {
      const int excl_unit = mode == kModeOneHot ? d.excl_tok / U.unit : -1;
      auto mass = [&](int u) -> double {  // unit u's mass in units of p
        double m = 0.0;
        if (u < U.units) {
          for (int k = 0; k < U.pper && u * U.pper + k < nparts; ++k) {
            const RowStat st = ps[u * U.pper + k];
            if (st.o != -INFINITY) m += st.s * static_cast<double>(exp2_fast(st.o - d.Ot));
          }
          m /= d.St;
          if (u == excl_unit) m = fmax(0.0, m - static_cast<double>(d.p_excl));
        }
        return m;
      };
      double carry = 0.0;
      for (int r = 0; r < rounds; ++r) carry = lane_broadcast(wave_inclusive_scan(mass(64 * r + lane)) + carry, 63);
      const double W = carry;
      if (!(W > 0.0) && mode == kModeOneHot) {  // all of the row's mass sat on the drafted token
        mode = kModeFallbackP;
        continue;
      }
      const double tt = static_cast<double>(d.uf) * W;
      int usel = -1, lastu = -1;
      double before = 0.0, last_before = 0.0;
      carry = 0.0;
      for (int r = 0; r < rounds && usel < 0; ++r) {
        const double m = mass(64 * r + lane);
        const double incl = wave_inclusive_scan(m) + carry;  // as for the total above
        carry = lane_broadcast(incl, 63);
        const unsigned long long hit = __ballot(m > 0.0 && incl >= tt);
        if (hit) {
          const int l = __ffsll(static_cast<long long>(hit)) - 1;
          usel = 64 * r + l;
          before = lane_broadcast(incl - m, l);
        }
        const unsigned long long pos = __ballot(m > 0.0);
        if (pos) {
          const int l = 63 - __clzll(static_cast<long long>(pos));
          lastu = 64 * r + l;
          last_before = lane_broadcast(incl - m, l);
        }
      }
      if (usel < 0) {  // rounding left u * W above every prefix: the last unit with mass
        usel = lastu >= 0 ? lastu : 0;
        before = lastu >= 0 ? last_before : 0.0;
      }
      if (lane == 0) {
        s_unit = usel;
        s_tu = tt - before;
        s_mode = mode;
      }
      break;
    }
  }
  __syncthreads();
  *usel_out = s_unit;
  *tunit_out = s_tu;
  *mode_io = s_mode;
}

// Step 2 for one segment held by the calling wave (v[j], lane l: the segment's vector
// l + 64 j; e0 = the segment's first element + l * E): per-vector fp32 sums of the draw
// weights (vs) and their inclusive fp64 prefixes in vocabulary order (incl); returns the
// segment's mass.
template <int DT>
__device__ __forceinline__ double wave_segment_scan(const ChainDecision& d, const u32x4 (&v)[kThreads / 64], int e0,
                                                    int excl, float (&vs)[kThreads / 64],
                                                    double (&incl)[kThreads / 64]) {
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  double carry = 0.0;
#pragma unroll
  for (int j = 0; j < kThreads / 64; ++j) {
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) sum += draw_weight(false, d, EL::get(v[j], i), 0.f, e0 + j * 64 * E + i, excl);
    vs[j] = sum;
    incl[j] = wave_inclusive_scan(static_cast<double>(sum)) + carry;
    carry = lane_broadcast(incl[j], 63);
  }
  return carry;
}

// Step 3's choice of segment among a unit's `segs` segment masses m[0..segs) (t_unit: u * W
// minus the mass before the unit): the first whose prefix reaches t_unit, else (rounding) the
// last with mass, else the first.  *qbase: the mass before it.
template <class Masses>
__device__ __forceinline__ int pick_segment(const Masses& m, int segs, double t_unit, double* qbase) {
  int q = -1, lastq = -1;
  double base = 0.0, lastbase = 0.0, run = 0.0;
  for (int k = 0; k < segs; ++k) {
    const double sm = m(k);
    if (sm > 0.0) {
      lastq = k;
      lastbase = run;
      if (q < 0 && run + sm >= t_unit) {
        q = k;
        base = run;
      }
    }
    run += sm;
  }
  if (q < 0) {
    q = lastq >= 0 ? lastq : 0;
    base = lastq >= 0 ? lastbase : 0.0;
  }
  *qbase = base;
  return q;
}

// Step 3's narrowing by the wave holding the segment (its scan from wave_segment_scan; t_seg:
// u * W minus the mass before the segment); returns the drawn element in every lane.
template <int DT>
__device__ __forceinline__ int wave_segment_pick(const ChainDecision& d, const u32x4 (&v)[kThreads / 64], int e0,
                                                 int excl, const float (&vs)[kThreads / 64],
                                                 const double (&incl)[kThreads / 64], double t_seg, int seg) {
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr int kSeg = ChunkShape<DT, 1>::kSegment;
  constexpr int kVPL = kThreads / 64;
  const int lane = threadIdx.x & 63;
  int jsel = -1, lsel = -1;
#pragma unroll
  for (int j = 0; j < kVPL; ++j) {
    const unsigned long long hit = __ballot(vs[j] > 0.f && incl[j] >= t_seg);
    if (jsel < 0 && hit) {
      jsel = j;
      lsel = __ffsll(static_cast<long long>(hit)) - 1;
    }
  }
  if (jsel < 0) {  // rounding left t_seg above the segment's total: its last positive weight
    int last_pos = -1;
#pragma unroll
    for (int j = 0; j < kVPL; ++j)
#pragma unroll
      for (int i = 0; i < E; ++i)
        if (draw_weight(false, d, EL::get(v[j], i), 0.f, e0 + j * 64 * E + i, excl) > 0.f)
          last_pos = max(last_pos, e0 + j * 64 * E + i);
    const int y = wave_max_int(last_pos);
    return y < 0 ? seg * kSeg : y;
  }
  int pick = -1;
  if (lane == lsel) {
    // (each vector walked under its own test, so that no vector is selected by a run-time
    // index, which would put the wave's vectors in scratch memory)
#pragma unroll
    for (int j = 0; j < kVPL; ++j)
      if (j == jsel) {
        double run = incl[j] - static_cast<double>(vs[j]);
        const int ev = e0 + j * 64 * E;
        int lastw = -1;
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const float wv = draw_weight(false, d, EL::get(v[j], i), 0.f, ev + i, excl);
          run += static_cast<double>(wv);
          if (wv > 0.f) lastw = ev + i;
          if (pick < 0 && wv > 0.f && run >= t_seg) pick = ev + i;
        }
        if (pick < 0) pick = lastw;
      }
  }
  return lane_broadcast(pick, lsel);
}

// The emitted row of sequence b after n accepted drafts xs[0..n) and the drawn token y
// (then -1), written by the lanes of one wave.
__device__ __forceinline__ void write_row_wave(const ChainArgs& a, int b, int n, const int32_t* xs, int y) {
  int32_t* ot = a.out_tokens + static_cast<size_t>(b) * (a.K + 1);
  for (int kk = static_cast<int>(threadIdx.x & 63); kk <= a.K; kk += 64) ot[kk] = kk < n ? xs[kk] : (kk == n ? y : -1);
}

// The whole direct draw by one workgroup, reading the unit's segments from memory; every lane
// calls it.  ps: the partials of row d.row; xs: the sequence's drafted tokens.
template <int DT, bool VEC>
__device__ __forceinline__ void direct_draw(const ChainArgs& a, int b, const ChainDecision& d, int mode,
                                            const void* row, const RowStat* ps, const int32_t* xs, size_t sb) {
  __shared__ double s_segm[kWaves];
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr int kSeg = ChunkShape<DT, 1>::kSegment;
  constexpr int kVPL = kThreads / 64;  // vectors of a segment per lane of a wave
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int usel;
  double t_unit;
  direct_locate<DT>(a, b, d, &mode, ps, &usel, &t_unit);
  stamp(a, sb + kPhPublished);
  const int excl = mode == kModeOneHot ? d.excl_tok : -1;
  const int segs = direct_units<DT>(a.nv, a.V).segs;

  // ---- 2. wave q: segment q of the unit, scanned in vocabulary order
  const int seg = usel * segs + w;  // this wave's segment
  const int e0 = seg * kSeg + lane * E;
  u32x4 v[kVPL];
  float vs[kVPL];
  double incl[kVPL];
  if (w < segs) {
#pragma unroll
    for (int j = 0; j < kVPL; ++j) v[j] = load_vector<DT, VEC>(row, a.V, e0 + j * 64 * E);
    const double m = wave_segment_scan<DT>(d, v, e0, excl, vs, incl);
    if (lane == 0) s_segm[w] = m;
  }
  __syncthreads();

  // ---- 3. the segment (the same choice in every lane), then the wave holding it narrows
  double qbase;
  const int q = pick_segment([&](int k) { return s_segm[k]; }, segs, t_unit, &qbase);
  if (w != q) return;
  const int y = wave_segment_pick<DT>(d, v, e0, excl, vs, incl, t_unit - qbase, seg);
  write_row_wave(a, b, d.n, xs, y);
}

// Outcomes of a residual draw's hand-over (slot_select, gather_and_locate).
enum SlotOutcome : int { kSlotDone = 0, kSlotLocated = 1, kSlotNoMass = 2 };

// Flags sequence b after a wait that gave up: -1 tokens, zero probabilities and the count
// kFlagTimedOut, written by threads first, first + step, ... (a whole workgroup or one wave; the
// one with first = 0 writes the count).
__device__ __forceinline__ void write_timed_out(const ChainArgs& a, int b, int first, int step) {
  int32_t* ot = a.out_tokens + static_cast<size_t>(b) * (a.K + 1);
  for (int kk = first; kk <= a.K; kk += step) ot[kk] = -1;
  if (a.out_probs)
    for (int i = first; i < a.K * 3; i += step) a.out_probs[static_cast<size_t>(b) * a.K * 3 + i] = 0.f;
  if (first == 0) a.out_num[b] = kFlagTimedOut;
}

// One wave alone (the other waves of its workgroup wait at a barrier): lane l takes segments
// l, l + 64, ... (round r holds segments 64 r .. 64 r + 63), waits for their masses, and the
// rounds' inclusive scans in vocabulary order give the total W and the segment whose prefix
// first reaches uf * W.  The masses stay in shared memory (s_m, room for S doubles); the scans
// are recomputed for the search.  Returns kSlotLocated with the segment and u * W minus the
// mass before it in *usel_out and *tloc_out (lane 0 writes them); kSlotNoMass if rounding
// left no residual mass (W = 0); kSlotDone if a wait gave up (the sequence is then flagged)
// or if abort() (wave-uniform, asked between polls) said that another workgroup finishes the
// draw.
template <class Abort>
__device__ __forceinline__ int gather_and_locate(const ChainArgs& a, int b, uint32_t gen, const SlotDouble* mw,
                                                 int units, float uf, double* s_m, int* usel_out, double* tloc_out,
                                                 size_t sb, Abort abort) {
  const int lane = threadIdx.x & 63;
  const int rounds = (units + 63) / 64;  // units = S <= 4 * kThreads
  {
    const SlotDouble* slots = mw;
    unsigned have = 0;  // rounds whose slot this lane has read
    for (int r = 0; r < rounds; ++r)
      if (64 * r + lane >= units) {
        have |= 1u << r;
        s_m[64 * r + lane] = 0.0;
      }
    const unsigned all = rounds >= 32 ? ~0u : (1u << rounds) - 1u;
    bool arrived = false;
    for (int polls = 0; polls < a.poll_limit; ++polls) {
      for (int r = 0; r < rounds; ++r) {
        double v;
        if (!(have >> r & 1u) && get_slot(slots + 64 * r + lane, gen, &v)) {
          have |= 1u << r;
          s_m[64 * r + lane] = v;
        }
      }
      if (__ballot(have != all) == 0ull) {
        arrived = true;
        break;
      }
      if (abort()) return kSlotDone;  // another workgroup finishes the draw
      short_pause();
    }
    if (!arrived) {  // flag the sequence rather than wait on (this task alone writes its row)
      write_timed_out(a, b, lane, 64);
      return kSlotDone;
    }
  }
  double W = 0.0;
  for (int r = 0; r < rounds; ++r) W = lane_broadcast(wave_inclusive_scan(s_m[64 * r + lane]) + W, 63);
  stamp(a, sb + kPhGathered);
  if (!(W > 0.0)) return kSlotNoMass;  // no residual mass left after rounding: draw from p_n itself
  const double tt = static_cast<double>(uf) * W;
  int usel = -1, lastu = -1;
  double before = 0.0, last_before = 0.0, carry = 0.0;
  for (int r = 0; r < rounds && usel < 0; ++r) {
    const double mr = s_m[64 * r + lane];
    const double ir = wave_inclusive_scan(mr) + carry;  // as in the total above
    carry = lane_broadcast(ir, 63);
    const unsigned long long hit = __ballot(mr > 0.0 && ir >= tt);
    if (hit) {
      const int l = __ffsll(static_cast<long long>(hit)) - 1;
      usel = 64 * r + l;
      before = lane_broadcast(ir - mr, l);
    }
    const unsigned long long pos = __ballot(mr > 0.0);
    if (pos) {  // the last segment with mass so far
      const int l = 63 - __clzll(static_cast<long long>(pos));
      lastu = 64 * r + l;
      last_before = lane_broadcast(ir - mr, l);
    }
  }
  if (usel < 0) {  // rounding left u * W above every prefix: the last segment with mass
    usel = lastu >= 0 ? lastu : 0;
    before = lastu >= 0 ? last_before : 0.0;
  }
  if (lane == 0) {
    *usel_out = usel;
    *tloc_out = tt - before;
  }
  return kSlotLocated;
}

// Residual mass of one vector of a row pair: the sum over its E elements, in order, of
// max(0, p - q) in fp32.
template <int DT>
__device__ __forceinline__ float residual_vector_mass(const ChainDecision& d, const u32x4& vt, const u32x4& vd) {
  using EL = Elem<DT>;
  float aw = 0.f;
#pragma unroll
  for (int i = 0; i < EL::kPerVec; ++i) {
    const float pv = exp2_fast(fmaf(EL::get(vt, i), d.scale, -d.Ot)) * d.invSt;
    aw += fmaxf(0.f, pv - exp2_fast(fmaf(EL::get(vd, i), d.scale, -d.Od)) * d.invSd);
  }
  return aw;
}

// Masses of `nseg` consecutive segments from the per-vector masses red[q * kThreads + t] of
// segment q's vector t, in fp64 (one 16-lane row of the workgroup sums one segment: lane r
// adds vectors 16 r .. 16 r + 15 in order, then the row's inclusive sum), published in slots
// mw[0 .. nseg) with tag `gen`.  Every lane calls it; nseg <= kThreads / 16.
__device__ __forceinline__ void publish_segment_masses(const float* red, int nseg, SlotDouble* mw, uint32_t gen,
                                                       bool local = false) {
  const int q = threadIdx.x >> 4;  // q < nseg: segment q
  const int r = threadIdx.x & 15;
  double v = 0.0;
  if (q < nseg) {
    const float* src = red + q * kThreads + r * 16;
#pragma unroll
    for (int i = 0; i < 16; ++i) v += static_cast<double>(src[i]);
  }
  v = row16_inclusive_sum(v);
  if (q < nseg && r == 15) put_slot(mw + q, v, gen, local);
}

// Residual draw after a rejection against draft rows (see chain_pool_kernel, steps 1-3):
// this task's segment masses of max(0, p - q) go out through the slots; the sequence's last
// task waits for the others' and returns kSlotLocated with the segment holding u * W and
// u * W minus the mass before it, or kSlotNoMass if rounding left no residual mass.  Other
// tasks return kSlotDone, and so does a last task whose wait gave up (it flags the
// sequence).  `red` is shared memory of 2 * SPT * kThreads floats.  local: the sequence's tasks
// share this XCD, the masses go through its L2.
template <int DT, int SPT, bool VEC>
__device__ __forceinline__ int slot_select(const ChainArgs& a, int b, int c, bool last, const ChainDecision& d,
                                           const void* row_t, const void* row_d, float* red, int* usel_out,
                                           double* tloc_out, size_t sb, uint32_t gen, bool local) {
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr int kSeg = ChunkShape<DT, 1>::kSegment;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;

  // ---- 1. per-lane masses of this task's segments: max(0, p - q), one vector per lane
  {
    const int sbase = c * SPT * kSeg;  // first element of this task's segments
    u32x4 rt[SPT], rd[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) rt[j] = load_vector<DT, VEC>(row_t, a.V, sbase + (j * kThreads + tid) * E);
#pragma unroll
    for (int j = 0; j < SPT; ++j) rd[j] = load_vector<DT, VEC>(row_d, a.V, sbase + (j * kThreads + tid) * E);
#pragma unroll
    for (int j = 0; j < SPT; ++j) red[j * kThreads + tid] = residual_vector_mass<DT>(d, rt[j], rd[j]);
  }
  __syncthreads();
  // ---- 2. segment totals in fp64
  const int units = a.S;  // segment slots per row
  SlotDouble* mw = a.wseg + static_cast<size_t>(b) * units;
  publish_segment_masses(red, SPT, mw + c * SPT, gen, local);
  stamp(a, sb + kPhPublished);
  if (!last) return kSlotDone;
  __shared__ int s_outcome, s_usel;
  __shared__ double s_tloc;
  __syncthreads();  // every wave is done with `red`, which holds the gathered masses next
  if (w == 0) {
    const int o = gather_and_locate(a, b, gen, mw, units, d.uf, reinterpret_cast<double*>(red), &s_usel, &s_tloc,
                                    sb, [] { return false; });
    if (lane == 0) s_outcome = o;
  }
  __syncthreads();
  *usel_out = s_usel;
  *tloc_out = s_tloc;
  return s_outcome;
}

// Narrows a draw to one element of segment `usel` and writes the emitted row (x_0 .. x_{n-1},
// the drawn token, then -1); called by every lane.  Lane t takes the segment's vector t, sums
// its draw weights in fp32 exactly as the segment masses were summed and scans the sums in
// fp64; the first lane whose prefix reaches t_loc picks the element, walking its weights in
// order, and writes it.  If rounding leaves t_loc above the segment's total, the last
// positive weight is taken; with no positive weight at all (a direct draw whose piece mass
// came from the stats partials while every weight underflows) the segment's first element.
// xs: the sequence's drafted tokens.  The segment's vectors come from memory, or from shared
// memory (st, sd: vector t at index t) where a caller holds them already.
template <int DT, bool VEC>
__device__ __forceinline__ void narrow_and_emit(const ChainArgs& a, int b, const ChainDecision& d, int mode,
                                                int usel, double t_loc, const void* row_t, const void* row_d,
                                                const int32_t* xs, const u32x4* st = nullptr,
                                                const u32x4* sd = nullptr) {
  __shared__ double s_wt[kWaves];
  __shared__ int s_first[kWaves];
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr int kSeg = ChunkShape<DT, 1>::kSegment;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const bool residual = mode == kModeResidual;
  const int excl = mode == kModeOneHot ? d.excl_tok : -1;
  const int e0 = usel * kSeg + tid * E;
  const u32x4 vt = st ? st[tid] : load_vector<DT, VEC>(row_t, a.V, e0);
  const u32x4 vd = !residual ? vt : (sd ? sd[tid] : load_vector<DT, VEC>(row_d, a.V, e0));
  float wl[E];
  float lsum = 0.f;
  int last_pos = -1;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    wl[i] = draw_weight(residual, d, EL::get(vt, i), EL::get(vd, i), e0 + i, excl);
    lsum += wl[i];
    last_pos = wl[i] > 0.f ? e0 + i : last_pos;
  }
  const double incl = wave_inclusive_scan(static_cast<double>(lsum));
  if (lane == 63) s_wt[w] = incl;
  __syncthreads();
  double lbefore = incl - static_cast<double>(lsum);
  for (int i = 0; i < w; ++i) lbefore += s_wt[i];
  const unsigned long long hit = __ballot(lsum > 0.f && lbefore + static_cast<double>(lsum) >= t_loc);
  if (lane == 0) s_first[w] = hit ? w * 64 + __ffsll(static_cast<long long>(hit)) - 1 : INT_MAX;
  __syncthreads();
  int kmin = s_first[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) kmin = min(kmin, s_first[i]);
  const int n = d.n;
  int32_t* ot = a.out_tokens + static_cast<size_t>(b) * (a.K + 1);
  if (kmin == INT_MAX) {  // rounding left t_loc above the segment total: last positive weight
    int y = block_max_int(last_pos, s_first);
    if (y < 0) y = usel * kSeg;
    for (int kk = tid; kk <= a.K; kk += kThreads) ot[kk] = kk < n ? xs[kk] : (kk == n ? y : -1);
    return;
  }
  for (int kk = tid; kk <= a.K; kk += kThreads)
    if (kk != n) ot[kk] = kk < n ? xs[kk] : -1;
  if (tid == kmin) {
    double run = lbefore;
    int pick = -1;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      run += wl[i];
      if (pick < 0 && wl[i] > 0.f && run >= t_loc) pick = e0 + i;
    }
    ot[n] = pick >= 0 ? pick : last_pos;
  }
}

// grid = Bs x CP pool tasks for the sequences b0 .. b0+Bs-1 (CP per sequence, below):
// task t = (sequence b, group c of SPT consecutive segments; a segment is one 16-byte vector
// per lane, 256*E elements, and a row has S segment slots, the last ones past V weighing 0).
//  1. Decides for b (identically in each of the sequence's tasks; the last task writes the
//     count and probabilities).  A bonus or one-hot draw is finished by the sequence's
//     first task alone (direct_draw); after a rejection against draft rows each task loads
//     its segments of the row pair and sums, for each segment, max(0, p - q): per lane in
//     fp32, across lanes in fp64.
//  2. Hands the segment masses over; the sequence's last task waits for those of its
//     siblings.
//  3. The last task scans the S segment masses in vocabulary order and takes the first
//     segment whose inclusive prefix reaches u * W (W = the total), narrows it to a lane
//     and an element and writes the emitted row (x_0 .. x_{n-1}, the drawn token, then
//     -1).  If rounding leaves no residual mass (W = 0 after a rejection) the last task
//     draws from p (the target row) as a bonus draw does.
// Only a sequence's last task waits, and only for tasks of the same launch that come before
// it in dispatch order and never wait themselves, so every wait ends even when other
// kernels share the device.  The host also keeps a launch to at most half as many sequences
// (hence waiting tasks) as pool workgroups fit at once, so the tasks waited for find room
// quickly.  Each wait is bounded besides: after the poll limit the last task flags the
// sequence -2 (it alone writes the sequence's count, probabilities and row, so the flag
// never mixes with a result).  (Measured at B=64, K=5, V=128256 bf16: letting every task
// wait, so that the task holding the drawn segment finishes with it still in cache, gave the
// same pool time, 14.5 us per call.)
//
// Tasks per sequence: CP = S / SPT when draft rows are given, else 1 (without draft rows every
// sampled draw is a bonus or one-hot draw from a target row's piece masses, which the first
// task finishes alone).  Workgroups go sequence by sequence, so a waiting task (a last task)
// comes after every task it waits for.
//
// Vocabulary order inside a chunk is segment-major (a segment = one 16-byte vector per
// lane), then lane, then element.
template <int DT, int SPT, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_pool_kernel(ChainArgs a, int b0, int CP) {
  constexpr int kRedBytes = 2 * SPT * kThreads * static_cast<int>(sizeof(float));
  __shared__ __align__(16) unsigned char s_buf[kRedBytes];
  __shared__ ChainDecision s_dec;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int gi = static_cast<int>(blockIdx.x);
  // Task ti of the launch, sequence-major.  With xcd_local and a multiple of 8 sequences in the
  // launch, XCD x (grid index mod 8) runs the tasks of sequences [x nb/8, (x+1) nb/8) of its nb,
  // each sequence's in task order, and their masses go through its L2.
  const int nb = static_cast<int>(gridDim.x) / CP;
  const bool place = a.xcd_local && nb % kXcds == 0;
  const int ti = place ? (gi % kXcds) * (nb / kXcds) * CP + gi / kXcds : gi;
  const bool local = place && on_indexed_xcd();
  const int b = b0 + ti / CP;  // sequence
  const int c = ti % CP;       // this task's group of SPT segments
  const bool last = c == CP - 1;
  float* red = reinterpret_cast<float*>(s_buf);  // [2][SPT][kThreads] per-lane masses
  const size_t sb = a.stamps_pool + kStampsPerTask * (static_cast<size_t>(b0) * CP + ti);
  stamp(a, sb + kPhStart);

  if (a.decided) {  // decided by chain_decide_kernel, which also wrote the count and probabilities
    if (tid == 0) s_dec = a.decs[b];
    __syncthreads();
  } else {
    chain_decide<DT>(a, b, clamped_len(a, b), seq_inputs(a, b), last, &s_dec);
  }
  const ChainDecision d = uniform_decision(s_dec);
  stamp(a, sb + kPhDecided);
  if (a.stamps && tid == 0)
    a.stamps[sb + kPhInfo] = (static_cast<unsigned long long>(b) << 32) | (static_cast<unsigned>(c) << 8) |
                             static_cast<unsigned>(d.mode);
  if (d.mode == kModeInvalid || d.mode == kModeGreedy) {  // the decision wrote the row
    stamp(a, sb + kPhEnd);
    return;
  }
  int mode = d.mode;
  const void* row_t = target_row<DT>(a, b, d.row);
  if (mode == kModeResidual) {
    int usel;
    double t_loc;
    // the slot generation is read after the decision, off its critical path (measured: 0.5 us
    // less pool time at B=64, K=5, V=128256; 2.3 us at B=256, K=8, V=152064)
    const int o = slot_select<DT, SPT, VEC>(a, b, c, last, d, row_t, draft_row<DT>(a, b, d.row), red, &usel, &t_loc,
                                            sb, pool_generation(a), local);
    if (o == kSlotLocated)
      narrow_and_emit<DT, VEC>(a, b, d, mode, usel, t_loc, row_t, draft_row<DT>(a, b, d.row),
                               a.tokens + static_cast<size_t>(b) * a.K);
    if (o != kSlotNoMass) {
      stamp(a, sb + kPhEnd);
      return;
    }
    mode = kModeFallbackP;  // no residual mass left after rounding: the last task draws from p_n
  } else if (c != 0) {      // a bonus or one-hot draw: the sequence's first task draws alone
    stamp(a, sb + kPhEnd);
    return;
  }
  direct_draw<DT, VEC>(a, b, d, mode, row_t, a.part + (static_cast<size_t>(b) * a.R + d.row) * a.C * kWaves,
                       a.tokens + static_cast<size_t>(b) * a.K, sb);
  stamp(a, sb + kPhEnd);
}

// grid = B: sequence b's decision, as chain_pool_kernel's tasks would each take it, once, for the
// pool kernel that follows (which then only reads it): count, probabilities and a -1 row for
// invalid input written here.  Used where a sequence has several pool tasks (draft rows given):
// at B=256, K=8, V=152064 the 4864 tasks, 1792 of them resident at a time, each combined the
// sequence's 340 partials before it could start its draw.
template <int DT>
__global__ __launch_bounds__(kThreads) void chain_decide_kernel(ChainArgs a) {
  __shared__ ChainDecision s_dec;
  const int b = static_cast<int>(blockIdx.x);
  chain_decide<DT>(a, b, clamped_len(a, b), seq_inputs(a, b), true, &s_dec);
  if (threadIdx.x == 0) a.decs[b] = s_dec;
}

// ---------------------------------------------------------------- single-launch path
//
// For batches whose whole grid fits on the device at once, one launch holds (in dispatch
// order) the n-gram lookup's workgroups (when it drafts) and then, sequence by sequence, one
// workgroup per position k = 0..K and chunk c.  That workgroup reads chunk c of target row k
// and, where a draft row scores position k, of draft row k, keeps both in registers, and
// publishes their wave partials (o, s) as words tagged with seq_tag.  It then gathers every
// partial its sequence's decision reads into shared memory and decides (every workgroup of the
// sequence reaches the same decision from the same data in the same order), and the
// workgroups of the draw's position finish the draw from their registers:
//  - a bonus or one-hot draw: the unit holding u * W is found from the partials
//    (direct_locate); the one wave holding that unit narrows it (wave_segment_scan,
//    pick_segment, wave_segment_pick);
//  - a residual draw: each workgroup of position n sums max(0, p - q) over its segments and
//    publishes the masses; each then gathers all of the row's masses and locates the segment
//    holding u * W (gather_and_locate), and the workgroup holding that segment stages it in
//    shared memory and narrows it (narrow_and_emit).
// The reads and the arithmetic are those of the separate launches (chain_stats_kernel, then
// chain_pool_kernel) with the same chunk size, so the two give the same outputs bit for bit.
//
// Waits.  The sequence's last workgroup (the anchor: position K, last chunk) waits only for
// workgroups dispatched before it, with the long poll limit; it writes the count and the
// probabilities.  The others wait for the partials with a short limit (kShortPolls) and
// publish a status word once they hold every partial (kStPassed) or gave up (kStLeft); one
// that passed never gives up afterwards.  The anchor checks the statuses of the workgroups
// the draw needs (the owner of a direct draw's unit; every workgroup of a residual draw's
// position): if any left, it finishes the draw itself from memory, as chain_pool_kernel does,
// and the workgroups of that position that passed see the departure and stand down.  So
// every wait ends (the long ones wait only for earlier workgroups, whose own waits are
// bounded), and exactly one workgroup writes each sequence's emitted row.  The anchor
// advances the sequence's run counter once every workgroup of the sequence has published
// its status (and so has read the counter).  If the anchor's own wait gives up and no
// workgroup passed, it flags the sequence -2.

constexpr int kPoolSegments = 4;       // segments per pool task (chain_pool_kernel)
constexpr int kSingleVectors = 4;      // vectors a lane in a chunk of the single launch
constexpr int kSingleMaxParts = 512;   // partials one sequence's decision reads (R * C * kWaves)
constexpr int kSingleMaxGroups = 1024; // workgroups of a single launch (about four per compute unit)
constexpr int kSmallTile = 1024;       // the lookup's context tile inside a shared launch (4 KiB)
constexpr int kShortPolls = 2048;      // polls of a non-anchor workgroup's wait for the partials
constexpr uint32_t kFallbackTagMix = 0x27d4eb2fu;  // slot tag of the anchor's own residual draw
enum SeqStatus : uint32_t { kStPassed = 1, kStLeft = 2 };

// Gather sequence b's decision inputs into shared memory; every lane calls it.  With the
// lookup (NGRAM) its draft length, tokens and their logits come as tagged words; otherwise
// the caller left them in s_kb, s_tok and s_gath before the call.  False if the wait gave up
// after `limit` polls.
__device__ __forceinline__ bool single_gather(const ChainArgs& a, int b, uint32_t tag, bool greedy, bool NGRAM,
                                              int limit, RowStat* s_part, int32_t* s_tok, float* s_gath,
                                              int* s_kb) {
  const int tid = threadIdx.x;
  const int C4 = a.C * kWaves;
  if (NGRAM) {
    const uint64_t* w = a.tprop + static_cast<size_t>(b) * (2 * a.K + 1);
    bool ok = false;
    for (int polls = 0; polls < limit; ++polls) {
      uint32_t v = 0;
      const bool got = tid != 0 || get_tagged_u32(w, tag, &v);
      if (tid == 0 && got) *s_kb = static_cast<int>(v);
      if (!__syncthreads_or(!got)) {
        ok = true;
        break;
      }
      short_pause();
    }
    if (!ok) return false;
    const int len = *s_kb;
    ok = false;
    for (int polls = 0; polls < limit; ++polls) {
      bool missing = false;
      if (tid < len) {
        uint32_t x = 0, g = 0;
        const bool hx = get_tagged_u32(w + 1 + tid, tag, &x);  // both reads go out before either is checked
        const bool hg = get_tagged_u32(w + 1 + a.K + tid, tag, &g);
        if (hx && hg) {
          s_tok[tid] = static_cast<int32_t>(x);
          s_gath[tid] = __uint_as_float(g);
        } else {
          missing = true;
        }
      }
      if (!__syncthreads_or(missing)) {
        ok = true;
        break;
      }
      short_pause();
    }
    if (!ok) return false;
  } else {
    __syncthreads();
  }
  const int kb_raw = *s_kb;
  const int kb = kb_raw < 0 ? 0 : (kb_raw > a.K ? a.K : kb_raw);
  // partials of the rows the decision reads (the lookup's case: every target row)
  const uint64_t* tp = a.tpart + static_cast<size_t>(b) * a.tstride;
  const int items = a.R * C4;
  unsigned have = 0;  // items tid, tid + kThreads (items <= kSingleMaxParts = 2 * kThreads)
  for (int polls = 0; polls < limit; ++polls) {
    bool missing = false;
#pragma unroll
    for (int j = 0; j < kSingleMaxParts / kThreads; ++j) {
      const int i = tid + j * kThreads;
      if (i < items && !(have >> j & 1u)) {
        if (!(NGRAM || row_needed(a, i / C4, kb, greedy))) {
          have |= 1u << j;
          continue;
        }
        uint32_t o;
        double sv;
        const bool ho = get_tagged_u32(tp + 3 * i, tag, &o);  // all three reads go out before any is checked
        const bool hs = get_tagged_double(tp + 3 * i + 1, tag, &sv);
        if (ho && hs) {
          s_part[i] = RowStat{__uint_as_float(o), 0.f, sv};
          have |= 1u << j;
        } else {
          missing = true;
        }
      }
    }
    if (!__syncthreads_or(missing)) return true;
    short_pause();
  }
  return false;
}

// Copies row `row`'s partials (published before the decision that led here) back into shared
// memory, every word checked against the tag (a bounded wait, for a reader that did not gather
// them itself); false if a wait gave up.  Every lane.
__device__ __forceinline__ bool single_restage_row(const ChainArgs& a, int b, uint32_t tag, int row, RowStat* s_part) {
  const int C4 = a.C * kWaves;
  const uint64_t* tp = a.tpart + static_cast<size_t>(b) * a.tstride + 3 * static_cast<size_t>(row) * C4;
  for (int polls = 0; polls < a.poll_limit; ++polls) {
    bool missing = false;
    for (int i = threadIdx.x; i < C4; i += kThreads) {
      uint32_t o = 0;
      double sv = 0.0;
      const bool ho = get_tagged_u32(tp + 3 * i, tag, &o);  // both reads go out before either is checked
      const bool hs = get_tagged_double(tp + 3 * i + 1, tag, &sv);
      missing |= !(ho && hs);
      s_part[static_cast<size_t>(row) * C4 + i] = RowStat{__uint_as_float(o), 0.f, sv};
    }
    if (!__syncthreads_or(missing)) return true;
    short_pause();
  }
  return false;
}

// The wave holding unit `usel` of a direct draw in registers (raw: this wave's share of the
// chunk, NV >= kWaves vectors a lane, so a unit is one wave's share) narrows it and writes the
// row; called by that wave alone.
template <int DT, int NV>
__device__ __forceinline__ void single_direct_finish(const ChainArgs& a, int b, const ChainDecision& d, int mode,
                                                     int usel, double t_unit, const u32x4 (&raw)[NV],
                                                     const int32_t* xs) {
  static_assert(NV >= kWaves, "a unit is one wave's share of a chunk");
  constexpr int E = Elem<DT>::kPerVec;
  constexpr int kSeg = ChunkShape<DT, 1>::kSegment;
  constexpr int kVPL = kThreads / 64;
  constexpr int kSegs = NV / kWaves;  // segments of the unit
  const int lane = threadIdx.x & 63;
  const int excl = mode == kModeOneHot ? d.excl_tok : -1;
  double m[kSegs];
#pragma unroll
  for (int q = 0; q < kSegs; ++q) {  // segment q: this wave's vectors 4q .. 4q + 3
    u32x4 v[kVPL];
    float vs[kVPL];
    double incl[kVPL];
#pragma unroll
    for (int j = 0; j < kVPL; ++j) v[j] = raw[q * kVPL + j];
    m[q] = wave_segment_scan<DT>(d, v, (usel * kSegs + q) * kSeg + lane * E, excl, vs, incl);
  }
  double qbase;
  const int q = pick_segment(
      [&](int k) {
        double r = m[0];
#pragma unroll
        for (int t = 1; t < kSegs; ++t)
          if (t == k) r = m[t];
        return r;
      },
      kSegs, t_unit, &qbase);
  u32x4 v[kVPL];
#pragma unroll
  for (int j = 0; j < kVPL; ++j) {
    v[j] = raw[j];
#pragma unroll
    for (int t = 1; t < kSegs; ++t)
      if (t == q) v[j] = raw[t * kVPL + j];
  }
  const int seg = usel * kSegs + q;
  const int e0 = seg * kSeg + lane * E;
  float vs[kVPL];
  double incl[kVPL];
  wave_segment_scan<DT>(d, v, e0, excl, vs, incl);
  const int y = wave_segment_pick<DT>(d, v, e0, excl, vs, incl, t_unit - qbase, seg);
  write_row_wave(a, b, d.n, xs, y);
}

// One workgroup of a single launch: sequence b, position k, chunk c (see above).
template <int DT, int NV, bool VEC, bool DRAFT>
__device__ __forceinline__ void single_task(const ChainArgs& a, int b, int k, int c, bool ngram) {
  using EL = Elem<DT>;
  constexpr size_t kBufBytes = kSingleMaxParts * sizeof(RowStat);
  constexpr int kMaxGroups = kSingleMaxParts / kWaves;  // workgroups of one sequence
  static_assert(2 * kThreads * sizeof(u32x4) <= kBufBytes, "a staged segment pair");
  static_assert(!DRAFT || NV * kThreads * sizeof(float) <= kBufBytes, "per-vector residual masses");
  static_assert(kMaxGroups <= kThreads, "one status a lane");
  __shared__ __align__(16) unsigned char s_buf[kBufBytes];  // partials; then masses or a staged segment
  __shared__ int32_t s_tok[SPEC_MAX_K];
  __shared__ float s_gath[2 * SPEC_MAX_K + 1];
  __shared__ float s_u[SPEC_MAX_K];
  __shared__ int s_kb;
  __shared__ ChainDecision s_dec;
  __shared__ int s_outcome, s_usel;
  __shared__ double s_tloc;
  __shared__ uint32_t s_stv[kMaxGroups];
  RowStat* s_part = reinterpret_cast<RowStat*>(s_buf);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int C = a.C;
  const int nw = (a.K + 1) * C;  // workgroups of the sequence
  const int j = k * C + c;
  const bool anchor = j == nw - 1;
  const int kb0 = ngram ? a.K : clamped_len(a, b);  // positions read: 0 .. kb0
  const bool greedy = is_greedy(a, b);
  const bool has_t = k <= kb0;
  if (!has_t && !anchor) return;  // reads nothing and takes no part
  const bool has_d = DRAFT && has_t && !greedy && k < kb0;
  const size_t sb = kStampsPerTask * (static_cast<size_t>(b) * nw + j);  // this workgroup's stamps
  stamp(a, sb + kSgStart);
  uint64_t* tp = a.tpart + static_cast<size_t>(b) * a.tstride;
  uint64_t* st = a.status + static_cast<size_t>(b) * a.sstride;
  const int S = a.S;
  const bool local = a.xcd_local && on_indexed_xcd();  // the sequence's workgroups share this XCD

  // the decision's scalar inputs and (wave 0, lane l) drafted token l and its uniform first,
  // then the chunks, then the tokens' logits
  const float T = input_load(a.temperature, b);
  const float uf = input_load(a.u_final, b);
  int x = -1;
  float ul = 1.f;
  if (w == 0 && lane < a.K) {
    if (!ngram) x = a.tokens[static_cast<size_t>(b) * a.K + lane];
    ul = a.u_accept[static_cast<size_t>(b) * a.K + lane];
  }
  u32x4 rt[NV], rd[NV];
  if (has_t) load_wave_span<DT, NV, VEC, true>(rt, target_row<DT>(a, b, k), a.V, c);
  if (has_d) load_wave_span<DT, NV, VEC, true>(rd, draft_row<DT>(a, b, k), a.V, c);
  uint32_t gt = 0u, gd = 0u;  // bits, converted when used
  if (!ngram && !greedy && w == 0 && lane < kb0 && x >= 0 && x < a.V) {
    gt = EL::bits(target_row<DT>(a, b, lane), x);
    if (DRAFT) gd = EL::bits(draft_row<DT>(a, b, lane), x);
  }
  // the tag's counter read goes out behind the chunks' loads (no load waits for it) and is
  // used once the partials are made
  const uint32_t run = load_agent(a.epoch + b);

  // this workgroup's partials
  const float scale = kLog2e / T;
  if (has_t) {
    float o;
    double sv;
    if (greedy) {
      int idx;
      wave_argmax_partial<DT, NV, VEC>(rt, c, a.V, &o, &idx);
      sv = static_cast<double>(idx);
    } else {
      wave_softmax_partial<DT, NV>(rt, scale, &o, &sv);
    }
    const uint32_t tg = seq_tag_from(a, run);
    const size_t i = (static_cast<size_t>(k) * C + c) * kWaves + w;
    if (lane == 0) {
      put_tagged_u32(tp + 3 * i, __float_as_uint(o), tg, local);
      put_tagged_double(tp + 3 * i + 1, sv, tg, local);
    }
  }
  if (has_d) {
    float o;
    double sv;
    wave_softmax_partial<DT, NV>(rd, scale, &o, &sv);
    const uint32_t tg = seq_tag_from(a, run);
    const size_t i = (static_cast<size_t>(a.K + 1 + k) * C + c) * kWaves + w;
    if (lane == 0) {
      put_tagged_u32(tp + 3 * i, __float_as_uint(o), tg, local);
      put_tagged_double(tp + 3 * i + 1, sv, tg, local);
    }
  }
  const uint32_t tag = seq_tag_from(a, run);
  stamp(a, sb + kSgPublished);

  // the decision's inputs
  if (w == 0) {
    if (lane < a.K) s_u[lane] = ul;
    if (!ngram) {
      if (lane < a.K) s_tok[lane] = x;
      if (lane < kb0) {
        s_gath[lane] = EL::from_bits(gt);
        if (DRAFT) s_gath[a.K + 1 + lane] = EL::from_bits(gd);
      }
      if (lane == 0) s_kb = a.draft_len ? input_load(a.draft_len, b) : a.K;
    }
  }
  const int limit = anchor ? a.poll_limit : min(a.poll_limit, kShortPolls);
  bool ok = single_gather(a, b, tag, greedy, ngram, limit, s_part, s_tok, s_gath, &s_kb);
  stamp(a, sb + kSgGathered);
  if (!anchor) {
    if (tid == 0) put_tagged_u32(st + j, ok ? kStPassed : kStLeft, tag, local);
    if (!ok) return;
  }
  // the anchor's view of the others: the sequence's other workgroups that read rows (its own
  // position, K, is among them only when it reads rows itself)
  const int others = min((kb0 + 1) * C, nw - 1);
  auto read_statuses = [&] {  // every lane; true once all are out (s_stv: the values, 0 = none)
    bool got = tid >= others;
    for (int polls = 0; polls < a.poll_limit; ++polls) {
      if (!got) {
        uint32_t v = 0;
        got = get_tagged_u32(st + tid, tag, &v);
        s_stv[tid] = got ? v : 0u;
      }
      if (!__syncthreads_or(!got)) return true;
      short_pause();
    }
    __syncthreads();
    return false;
  };
  if (!ok) {  // the anchor's wait gave up: go on if another workgroup holds every partial
    read_statuses();
    bool passed = false;
    for (int i = tid; i < others; i += kThreads) passed |= s_stv[i] == kStPassed;
    if (__syncthreads_or(passed)) ok = single_gather(a, b, tag, greedy, ngram, a.poll_limit, s_part, s_tok, s_gath, &s_kb);
    if (!ok) {
      write_timed_out(a, b, tid, kThreads);
      if (tid == 0) __hip_atomic_fetch_add(a.epoch + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }

  const int kb_raw = s_kb;
  const int kb = kb_raw < 0 ? 0 : (kb_raw > a.K ? a.K : kb_raw);
  SlotDouble* tm = a.tmass + static_cast<size_t>(b) * a.K * S;  // [K][S]
  // Before deciding, a workgroup whose position has draft rows publishes its segments' residual
  // masses for a rejection at its position (they need only that position's row offsets and
  // sums, with the arithmetic the decision would give them), so that they are out by the time
  // the decision is.
  auto speculate = [&](const float* sO, const double* sS) {
    if (!(has_d && k < kb)) return;
    ChainDecision dk{};
    dk.scale = scale;
    dk.Ot = sO[k];
    dk.invSt = static_cast<float>(inv_row_sum(sS[k]));
    dk.Od = sO[a.K + 1 + k];
    dk.invSd = static_cast<float>(inv_row_sum(sS[a.K + 1 + k]));
    float* red = reinterpret_cast<float*>(s_buf);  // the partials are combined: free
#pragma unroll
    for (int jv = 0; jv < NV; ++jv) red[(w * NV + jv) * 64 + lane] = residual_vector_mass<DT>(dk, rt[jv], rd[jv]);
    __syncthreads();
    // this chunk holds segments c * NV .. c * NV + NV - 1 (those from S on lie past V)
    publish_segment_masses(red, min(NV, S - c * NV), tm + static_cast<size_t>(k) * S + c * NV, tag, local);
  };
  chain_decide<DT>(a, b, kb, SeqInputs{s_part, s_tok, s_gath, s_u, T, uf, kb_raw}, anchor, &s_dec, speculate);
  const ChainDecision d = uniform_decision(s_dec);
  stamp(a, sb + kSgDecided);
  const int mode = d.mode;
  const int row = d.row;
  const bool direct = mode == kModeBonus || mode == kModeOneHot;
  int owner_c = -1;  // a direct draw: the chunk holding its unit
  if (mode == kModeResidual && DRAFT && k == row) {
    // every workgroup of position n has published its masses: gather them, locate the draw
    if (w == 0) {
      const int o = gather_and_locate(a, b, tag, tm + static_cast<size_t>(row) * S, S, d.uf,
                                      reinterpret_cast<double*>(s_buf), &s_usel, &s_tloc, kNoStamp, [&] {
                                        bool gone = false;
                                        if (lane < C) {
                                          uint32_t v = 0;
                                          gone = get_tagged_u32(st + row * C + lane, tag, &v) && v == kStLeft;
                                        }
                                        return __ballot(gone) != 0ull;
                                      });
      if (lane == 0) s_outcome = o;
    }
    __syncthreads();
    stamp(a, sb + kSgDrawn);
    const int o = s_outcome;
    if (o == kSlotLocated) {
      const int usel = s_usel;
      if (usel / NV != c) return;
      // stage the segment pair (vector t of the segment at index t) and narrow it
      u32x4* stt = reinterpret_cast<u32x4*>(s_buf);
      u32x4* sdd = stt + kThreads;
      const int sq = usel % NV;
#pragma unroll
      for (int jv = 0; jv < NV; ++jv) {
        const int tc = (w * NV + jv) * 64 + lane;  // vector index within the chunk
        if (tc / kThreads == sq) {
          stt[tc % kThreads] = rt[jv];
          sdd[tc % kThreads] = rd[jv];
        }
      }
      __syncthreads();
      narrow_and_emit<DT, VEC>(a, b, d, mode, usel, s_tloc, nullptr, nullptr, s_tok, stt, sdd);
      stamp(a, sb + kSgEnd);
      return;
    }
    if (o != kSlotNoMass) return;
    // no residual mass after rounding: the draw takes p_n itself, as a bonus draw would
    // (this workgroup gathered and checked these words itself, so the re-read finds them)
    (void)single_restage_row(a, b, tag, row, s_part);
    int m2 = kModeFallbackP, usel;
    double t_unit;
    direct_locate<DT>(a, b, d, &m2, s_part + static_cast<size_t>(row) * C * kWaves, &usel, &t_unit);
    if (usel / kWaves == c && w == usel % kWaves) single_direct_finish<DT, NV>(a, b, d, m2, usel, t_unit, rt, s_tok);
    return;
  }
  if (direct && (k == row || anchor)) {
    int m2 = mode, usel;
    double t_unit;
    direct_locate<DT>(a, b, d, &m2, s_part + static_cast<size_t>(row) * C * kWaves, &usel, &t_unit);
    stamp(a, sb + kSgDrawn);
    owner_c = usel / kWaves;  // a unit is one wave's share: four to a chunk
    if (k == row && c == owner_c && w == usel % kWaves) {
      single_direct_finish<DT, NV>(a, b, d, m2, usel, t_unit, rt, s_tok);
      if (a.stamps && lane == 0) a.stamps[sb + kSgEnd] = __builtin_amdgcn_s_memrealtime();
    }
  }
  if (!anchor) return;
  // The anchor: every status (also the one every workgroup's use of the run counter ends with);
  // a draw whose workgroups did not all pass is finished here from memory
  const bool all = read_statuses();
  if (direct && !(k == row && c == owner_c) && s_stv[row * C + owner_c] != kStPassed)
    direct_draw<DT, VEC>(a, b, d, mode, target_row<DT>(a, b, row), s_part + static_cast<size_t>(row) * C * kWaves,
                         s_tok, kNoStamp);
  if (mode == kModeResidual && DRAFT) {
    bool gone = false;
    for (int i = tid; i < C; i += kThreads) gone |= s_stv[row * C + i] != kStPassed;
    if (__syncthreads_or(gone)) {
      const void* row_t = target_row<DT>(a, b, row);
      const void* row_d = draft_row<DT>(a, b, row);
      const uint32_t g2 = tag ^ kFallbackTagMix;
      float* red = reinterpret_cast<float*>(s_buf);
      int usel = 0, o = kSlotDone;
      double t_loc = 0.0;
      for (int cg = 0; cg < S / kPoolSegments; ++cg)
        o = slot_select<DT, kPoolSegments, VEC>(a, b, cg, cg == S / kPoolSegments - 1, d, row_t, row_d, red, &usel,
                                                &t_loc, kNoStamp, g2, false);
      if (o == kSlotLocated) narrow_and_emit<DT, VEC>(a, b, d, mode, usel, t_loc, row_t, row_d, s_tok);
      if (o == kSlotNoMass) {
        (void)single_restage_row(a, b, tag, row, s_part);  // gathered and checked here before
        direct_draw<DT, VEC>(a, b, d, kModeFallbackP, row_t, s_part + static_cast<size_t>(row) * C * kWaves, s_tok,
                             kNoStamp);
      }
    }
  }
  (void)all;
  if (tid == 0) __hip_atomic_fetch_add(a.epoch + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  stamp(a, sb + kSgEnd);
}

// The n-gram lookup for sequence i inside a chain launch, through context tiles of TILE tokens
// in s_ctx (kTileInts<TILE> ints of shared memory): its draft length, tokens and their target
// logits go out as words tagged with seq_tag (and the lookup's outputs to the caller).
template <int DT, int TILE>
__device__ __forceinline__ void lookup_workgroup(const ChainArgs& a, const NgramArgs& ng, int i, int* s_ctx) {
  int32_t* tokens = const_cast<int32_t*>(a.tokens);
  const int len = ngram_propose_in<kThreads, TILE>(s_ctx, i, ng.context, ng.context_len, ng.L_max, ng.n_min, ng.n_max,
                                                   a.K, tokens, const_cast<int32_t*>(a.draft_len), ng.match_n);
  const uint32_t tag = seq_tag(a, i);
  const bool local = a.xcd_local && on_indexed_xcd();  // the sequence's workgroups share this XCD
  uint64_t* w = a.tprop + static_cast<size_t>(i) * (2 * a.K + 1);
  for (int k = threadIdx.x; k < len; k += kThreads) {  // lane k wrote token k above and reads it back
    const int x = tokens[static_cast<size_t>(i) * a.K + k];
    const float g = x >= 0 && x < a.V ? Elem<DT>::value(target_row<DT>(a, i, k), x) : 0.f;
    put_tagged_u32(w + 1 + k, static_cast<uint32_t>(x), tag, local);
    put_tagged_u32(w + 1 + a.K + k, __float_as_uint(g), tag, local);
  }
  if (threadIdx.x == 0) put_tagged_u32(w, static_cast<uint32_t>(len), tag, local);
}

// grid = P + B x (K+1) x C: P = B lookup workgroups when the lookup drafts (else 0), then the
// sequences' workgroups (position k, chunk c).  With xcd_local (batches of 8 or more),
// grid = 8 x ceil(B/8) x (L + (K+1) C) (L = 1 when the lookup drafts, else 0): XCD x (grid index
// mod 8) runs sequences x, x + 8, ..., first their lookups, then each sequence's workgroups in
// order, and the rest of its share idles, so that every hand-over of a sequence stays in one
// XCD's L2 (store_xcd).
template <int DT, int NV, bool VEC, bool DRAFT>
__global__ __launch_bounds__(kThreads) void chain_single_kernel(ChainArgs a, NgramArgs ng, int P) {
  __shared__ int s_ctx[kTileInts<kSmallTile>];
  const int per = (a.K + 1) * a.C;
  int i = static_cast<int>(blockIdx.x);
  if (a.xcd_local) {
    const int x = i % kXcds;
    int m = i / kXcds;
    const int nb = x < a.B ? (a.B - x + kXcds - 1) / kXcds : 0;  // sequences of XCD x
    if (P > 0) {
      if (m < nb) {
        lookup_workgroup<DT, kSmallTile>(a, ng, x + kXcds * m, s_ctx);
        return;
      }
      m -= nb;
    }
    if (m >= nb * per) return;  // beyond this XCD's share
    single_task<DT, NV, VEC, DRAFT>(a, x + kXcds * (m / per), (m % per) / a.C, m % a.C, P > 0);
    return;
  }
  if (i < P) {
    lookup_workgroup<DT, kSmallTile>(a, ng, i, s_ctx);
    return;
  }
  i -= P;
  const int j = i % per;
  single_task<DT, NV, VEC, DRAFT>(a, i / per, j / a.C, j % a.C, P > 0);
}

// ---------------------------------------------------------------- fused path
//
// Batches that do not run as a single launch run the statistics and the draw in one launch
// when each sequence's partials fit in kSingleMaxParts and its pool tasks in the status words:
// grid = G stats workgroups (in xcd_blocked chunk order, as chain_stats_kernel) and then CP
// helper workgroups per sequence (as chain_pool_kernel's tasks).  A stats workgroup publishes
// its wave partials as tagged words (seq_tag).  The sequence's stats workgroup dispatched
// last (its finisher) then gathers the sequence's partials, waiting only for workgroups
// dispatched before it, decides (writing the count and the probabilities), publishes the
// decision as tagged words and finishes a bonus or one-hot draw itself (direct_draw).  The
// helpers wait for the decision (nine words: cheaper to poll while the pass still streams than
// the partials, which they could decide from too; measured 44.2 against 42.6 us per call at
// B=64, K=5, V=128256); after a rejection against draft rows each sums max(0, p - q) over its
// segments and hands the masses over as chain_pool_kernel's tasks do, every helper locates the
// draw, and the one holding the drawn segment narrows it from its registers (no second read
// of the segment).  Every wait is on workgroups dispatched earlier whose own waits end, so every
// wait ends; the last helper advances the sequence's run counter once every helper has
// published that it read it (the finisher having read it before deciding, and every stats
// workgroup whose partials it gathered before publishing them).  A sequence is decided as
// soon as its own rows are summed, so the draws of the sequences finished early overlap the
// rest of the pass, and no launch boundary separates the pass from the draws.  The reads and
// arithmetic are those of the separate launches, whose outputs it gives bit for bit.

constexpr int kFusedDecisionWords = 9;
// Reads of a hand-over word kept in flight by a pipelined wait (a wait may make up to that many
// reads beyond its poll limit), and the pause between starting them (s_sleep 8: 512 clocks,
// about a quarter of a memory round trip at the end of the pass).
constexpr int kPollsInFlight = 4;
__device__ __forceinline__ void stagger_pause() { __builtin_amdgcn_s_sleep(8); }
// Helpers of one fused launch at most (beyond, the separate launches: measured at B=256, K=8,
// V=152064 bf16 with 4864 helpers, 234.7 us per call fused against 229.1 separate; at B=64,
// K=5, V=128256 with 1024, 43.9 against 44.5).
constexpr long long kFusedMaxHelpers = 2048;

// Dispatch index of chunk g in xcd_blocked order over G workgroups (its inverse).
__device__ __forceinline__ int xcd_blocked_inverse(int g, int G) {
  if (G % kXcds != 0) return g;
  const int blk = G / kXcds;
  return (g % blk) * kXcds + g / blk;
}

// Whether chunk g is the last dispatched of its sequence's chunks [g0, g1).
__device__ __forceinline__ bool last_dispatched(int g, int g0, int g1, int G) {
  if (G % kXcds != 0) return g == g1 - 1;
  const int blk = G / kXcds;
  int best = -1;
  for (int x = g0 / blk; x <= (g1 - 1) / blk; ++x)  // the sequence's last chunk in each XCD's block
    best = max(best, xcd_blocked_inverse(min(g1, (x + 1) * blk) - 1, G));
  return xcd_blocked_inverse(g, G) == best;
}

// A finisher's own decision inputs (wave 0, lane l: drafted token l, its accept uniform and
// the bits of its target and draft logits), fetched in two steps around the loads of its
// chunk so that the fetches overlap the chunk's streaming: first the tokens and scalars, then
// (once the chunk's loads are out) the logits at the tokens, converted only when used.
struct FinisherInputs {
  int x = -1;
  float ul = 1.f;
  uint32_t gt = 0u, gd = 0u;
  float T = 0.f, uf = 0.f;
  int kb_raw = 0;
};

__device__ __forceinline__ void finisher_fetch_tokens(const ChainArgs& a, int b, FinisherInputs* f) {
  const int lane = threadIdx.x & 63;
  f->T = input_load(a.temperature, b);
  f->uf = input_load(a.u_final, b);
  f->kb_raw = a.draft_len ? input_load(a.draft_len, b) : a.K;
  if (threadIdx.x < 64 && lane < a.K) {
    f->x = a.tokens[static_cast<size_t>(b) * a.K + lane];
    f->ul = a.u_accept[static_cast<size_t>(b) * a.K + lane];
  }
}

template <int DT>
__device__ __forceinline__ void finisher_fetch_logits(const ChainArgs& a, int b, int kb0, bool greedy,
                                                      FinisherInputs* f) {
  using EL = Elem<DT>;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64 && !greedy && lane < kb0 && f->x >= 0 && f->x < a.V) {
    f->gt = EL::bits(target_row<DT>(a, b, lane), f->x);
    if (a.draft) f->gd = EL::bits(draft_row<DT>(a, b, lane), f->x);
  }
}

// The finisher of sequence b (every lane): gathers, decides, publishes the decision and
// finishes a direct draw.  s_part: shared memory for kSingleMaxParts partials; f: its inputs
// as finisher_fetch_tokens and finisher_fetch_logits left them.
template <int DT, bool VEC>
__device__ __forceinline__ void fused_finish(const ChainArgs& a, int b, uint32_t tag, bool local, RowStat* s_part,
                                             const FinisherInputs& f) {
  __shared__ int32_t s_tok[SPEC_MAX_K];
  __shared__ float s_gath[2 * SPEC_MAX_K + 1];
  __shared__ float s_u[SPEC_MAX_K];
  __shared__ int s_kb;
  __shared__ ChainDecision s_dec;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kb0 = clamped_len(a, b);
  const bool greedy = f.T == 0.f;
  const float T = f.T;
  const float uf = f.uf;
  if (tid < 64) {
    if (lane < a.K) {
      s_tok[lane] = f.x;
      s_u[lane] = f.ul;
    }
    if (lane < kb0) {
      s_gath[lane] = Elem<DT>::from_bits(f.gt);
      if (a.draft) s_gath[a.K + 1 + lane] = Elem<DT>::from_bits(f.gd);
    }
    if (lane == 0) s_kb = f.kb_raw;
  }
  uint64_t* dw = a.tdec + static_cast<size_t>(b) * kFusedDecisionWords;
  const size_t fb = 2 * static_cast<size_t>(a.B) * a.R * a.C + kFinisherStamps * static_cast<size_t>(b);
  if (!single_gather(a, b, tag, greedy, false, a.poll_limit, s_part, s_tok, s_gath, &s_kb)) {
    // the wait gave up: flag the sequence (this workgroup alone writes its outputs) and let
    // the helpers stand down
    write_timed_out(a, b, tid, kThreads);
    if (tid < kFusedDecisionWords)
      put_tagged_u32(dw + tid, tid == 0 ? static_cast<uint32_t>(kModeInvalid) : 0u, tag, local);
    return;
  }
  stamp(a, fb + kFnGathered);
  const int kb_raw = s_kb;
  const int kb = kb_raw < 0 ? 0 : (kb_raw > a.K ? a.K : kb_raw);
  chain_decide<DT>(a, b, kb, SeqInputs{s_part, s_tok, s_gath, s_u, T, uf, kb_raw}, true, &s_dec);
  const ChainDecision d = uniform_decision(s_dec);
  if (tid < kFusedDecisionWords) {  // what a residual draw needs
    const uint64_t st_bits = static_cast<uint64_t>(__double_as_longlong(d.St));
    const uint32_t v[kFusedDecisionWords] = {
        static_cast<uint32_t>(d.mode) | (static_cast<uint32_t>(d.n) << 8) | (static_cast<uint32_t>(d.row) << 16),
        __float_as_uint(d.scale), __float_as_uint(d.Ot), __float_as_uint(d.invSt), __float_as_uint(d.Od),
        __float_as_uint(d.invSd), __float_as_uint(d.uf), static_cast<uint32_t>(st_bits),
        static_cast<uint32_t>(st_bits >> 32)};
    uint32_t mine = v[0];
#pragma unroll
    for (int i = 1; i < kFusedDecisionWords; ++i)
      if (i == tid) mine = v[i];
    put_tagged_u32(dw + tid, mine, tag, local);
  }
  stamp(a, fb + kFnDecided);
  if (d.mode == kModeBonus || d.mode == kModeOneHot)
    direct_draw<DT, VEC>(a, b, d, d.mode, target_row<DT>(a, b, d.row), s_part + static_cast<size_t>(d.row) * a.C * kWaves,
                         s_tok, kNoStamp);
  stamp(a, fb + kFnEnd);
  if (a.stamps && tid == 0) a.stamps[fb + kFnMode] = static_cast<unsigned long long>(d.mode);
}

// Stats workgroup for chunk g of a fused launch of G stats workgroups.  s_mem: the launch's
// shared buffer.
template <int DT, int NV, bool VEC>
__device__ __forceinline__ void fused_stats(const ChainArgs& a, int g, int G, unsigned char* s_mem) {
  const int c = g % a.C;
  const int rr = (g / a.C) % a.R;
  const int b = g / (a.C * a.R);
  const int kb = clamped_len<true>(a, b);
  const bool greedy = is_greedy<true>(a, b);
  const bool needed = row_needed(a, rr, kb, greedy);
  const int g0 = b * a.R * a.C;
  const bool finisher = last_dispatched(g, g0, g0 + a.R * a.C, G);
  if (!needed && !finisher) return;
  stamp(a, 2 * static_cast<size_t>(g));
  // the partials' readers (the finisher) and the decision's (the helpers) share this XCD
  const bool local = a.xcd_local && on_indexed_xcd();
  FinisherInputs f;
  if (finisher) finisher_fetch_tokens(a, b, &f);
  u32x4 raw[NV];
  if (needed) {
    const void* row = rr <= a.K ? target_row<DT>(a, b, rr) : draft_row<DT>(a, b, rr - (a.K + 1));
    load_wave_span<DT, NV, VEC, true>(raw, row, a.V, c);
  }
  if (finisher) finisher_fetch_logits<DT>(a, b, kb, greedy, &f);
  // the tag's counter read goes out behind the chunk's loads (no load waits for it) and is
  // used once the partials are made (the sums need not wait for it either)
  const uint32_t run = load_agent(a.epoch + b);
  uint32_t tag = 0u;
  if (needed) {
    float o;
    double sv;
    if (greedy) {
      int idx;
      wave_argmax_partial<DT, NV, VEC>(raw, c, a.V, &o, &idx);
      sv = static_cast<double>(idx);
    } else {
      wave_softmax_partial<DT, NV>(raw, kLog2e / input_load<true>(a.temperature, b), &o, &sv);
    }
    tag = seq_tag_from(a, run);
    if ((threadIdx.x & 63) == 0) {
      uint64_t* tp = a.tpart + static_cast<size_t>(b) * a.tstride +
                     3 * ((static_cast<size_t>(rr) * a.C + c) * kWaves + (threadIdx.x >> 6));
      put_tagged_u32(tp, __float_as_uint(o), tag, local);
      put_tagged_double(tp + 1, sv, tag, local);
    }
  }
  stamp(a, 2 * static_cast<size_t>(g) + 1);
  if (!finisher) return;
  fused_finish<DT, VEC>(a, b, seq_tag_from(a, run), local, reinterpret_cast<RowStat*>(s_mem), f);
}

// Helper c of CP for sequence b (every lane).
// s_buf: the launch's shared buffer (per-lane masses, then a staged segment pair, or row n's
// partials).
template <int DT, int SPT, bool VEC>
__device__ __forceinline__ void fused_helper(const ChainArgs& a, int b, int c, int CP, unsigned char* s_buf) {
  static_assert(2 * SPT * kThreads * sizeof(float) <= kSingleMaxParts * sizeof(RowStat), "buffer");
  __shared__ uint32_t s_w[kFusedDecisionWords];
  const int tid = threadIdx.x;
  const bool last = c == CP - 1;
  const size_t hb = 2 * static_cast<size_t>(a.B) * a.R * a.C + kFinisherStamps * static_cast<size_t>(a.B) +
                    kHelperStamps * (static_cast<size_t>(b) * CP + c);
  stamp(a, hb + kHpStart);
  const uint32_t tag = seq_tag(a, b);
  const bool local = a.xcd_local && on_indexed_xcd();  // the sequence's other helpers share this XCD
  uint64_t* st = a.status + static_cast<size_t>(b) * a.sstride;
  if (!last && tid == 0) put_tagged_u32(st + c, 1u, tag, local);  // this helper has read the run counter
  const uint64_t* dw = a.tdec + static_cast<size_t>(b) * kFusedDecisionWords;
  // Wave 0 waits for the decision words (lanes 0-8) with kPollsInFlight reads of each in flight,
  // started a quarter of a round trip apart and each reissued as soon as it returns, so that
  // the words are sampled four times a round trip rather than once; in the last helper, lanes
  // 9-63 watch the other helpers' status words meanwhile, so that advancing the run counter at
  // the end rarely needs another poll.  Each read counts as a poll.
  __shared__ int s_ok, s_nseen;
  if (tid < 64) {
    const bool dec_lane = tid < kFusedDecisionWords;
    const int si = tid - kFusedDecisionWords;  // status word this lane watches
    const bool st_lane = last && si >= 0 && si < CP - 1;
    const uint64_t* src = dec_lane ? dw + tid : (st_lane ? st + si : dw);
    bool got = false, st_seen = false;
    uint64_t took = 0;
    if (a.poll_limit > 0) {
      // (each read is reissued as soon as it is checked, even by the check that ends the wait,
      // and the limit is checked once a round: so the reads in flight stay in issue order and
      // each check waits for its own read alone)
      uint64_t r0 = load_agent(src);
      stagger_pause();
      uint64_t r1 = load_agent(src);
      stagger_pause();
      uint64_t r2 = load_agent(src);
      stagger_pause();
      uint64_t r3 = load_agent(src);
      auto step = [&](uint64_t& r) {
        const bool valid = static_cast<uint32_t>(r >> 32) == tag;
        st_seen |= st_lane && valid;
        const bool all = __ballot(dec_lane && !valid) == 0ull;
        if (all) took = r;
        got |= all;
        r = load_agent(src);
        return all;
      };
      for (int polls = kPollsInFlight; !(step(r0) || step(r1) || step(r2) || step(r3)) && polls < a.poll_limit;
           polls += kPollsInFlight) {
      }
    }
    if (got && dec_lane) s_w[tid] = static_cast<uint32_t>(took);
    const int nseen = __popcll(__ballot(st_seen));
    if (tid == 0) {
      s_ok = got ? 1 : 0;
      s_nseen = nseen;
    }
  }
  __syncthreads();
  const bool ok = s_ok != 0;
  stamp(a, hb + kHpSeen);
  if (ok && (uniform(static_cast<int>(s_w[0] & 0xff)) == kModeResidual)) {
    ChainDecision d{};
    d.mode = kModeResidual;
    d.n = uniform(static_cast<int>((s_w[0] >> 8) & 0xff));
    d.row = uniform(static_cast<int>((s_w[0] >> 16) & 0xff));
    d.excl_tok = -1;
    d.scale = uniform(__uint_as_float(s_w[1]));
    d.Ot = uniform(__uint_as_float(s_w[2]));
    d.invSt = uniform(__uint_as_float(s_w[3]));
    d.Od = uniform(__uint_as_float(s_w[4]));
    d.invSd = uniform(__uint_as_float(s_w[5]));
    d.uf = uniform(__uint_as_float(s_w[6]));
    d.St = uniform(__longlong_as_double(static_cast<long long>(
        (static_cast<uint64_t>(s_w[8]) << 32) | static_cast<uint64_t>(s_w[7]))));
    using EL = Elem<DT>;
    const void* row_t = target_row<DT>(a, b, d.row);
    const void* row_d = draft_row<DT>(a, b, d.row);
    const int32_t* xs = a.tokens + static_cast<size_t>(b) * a.K;
    // this helper's segments c * SPT .. c * SPT + SPT - 1 (lane t: vector t of each), their
    // masses as chain_pool_kernel's tasks sum them
    constexpr int kSeg = ChunkShape<DT, 1>::kSegment;
    float* red = reinterpret_cast<float*>(s_buf);
    u32x4 rt[SPT], rd[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) rt[j] = load_vector<DT, VEC>(row_t, a.V, (c * SPT + j) * kSeg + tid * EL::kPerVec);
#pragma unroll
    for (int j = 0; j < SPT; ++j) rd[j] = load_vector<DT, VEC>(row_d, a.V, (c * SPT + j) * kSeg + tid * EL::kPerVec);
#pragma unroll
    for (int j = 0; j < SPT; ++j) red[j * kThreads + tid] = residual_vector_mass<DT>(d, rt[j], rd[j]);
    __syncthreads();
    SlotDouble* mw = a.wseg + static_cast<size_t>(b) * a.S;
    publish_segment_masses(red, SPT, mw + c * SPT, tag, local);
    stamp(a, hb + kHpPublished);
    __syncthreads();  // `red` holds the gathered masses next
    // every helper gathers the masses and locates the draw; the one holding the segment
    // narrows it from its registers
    __shared__ int s_outcome, s_usel;
    __shared__ double s_tloc;
    if (tid < 64) {
      const int o = gather_and_locate(a, b, tag, mw, a.S, d.uf, reinterpret_cast<double*>(s_buf), &s_usel, &s_tloc, kNoStamp,
                                      [] { return false; });
      if (tid == 0) s_outcome = o;
    }
    __syncthreads();
    stamp(a, hb + kHpLocated);
    const int o = s_outcome;
    if (a.stamps && tid == 0)
      a.stamps[hb + kHpInfo] = (static_cast<unsigned long long>(b) << 32) | (static_cast<unsigned>(c) << 8) |
                               static_cast<unsigned>(o == kSlotLocated && s_usel / SPT == c ? 1 : 0);
    if (o == kSlotLocated && s_usel / SPT == c) {
      const int q = s_usel % SPT;
      u32x4* stt = reinterpret_cast<u32x4*>(s_buf);
      u32x4* sdd = stt + kThreads;
      u32x4 vt = rt[0], vd = rd[0];
#pragma unroll
      for (int j = 1; j < SPT; ++j)
        if (j == q) {
          vt = rt[j];
          vd = rd[j];
        }
      stt[tid] = vt;
      sdd[tid] = vd;
      __syncthreads();
      narrow_and_emit<DT, VEC>(a, b, d, d.mode, s_usel, s_tloc, row_t, row_d, xs, stt, sdd);
      stamp(a, hb + kHpNarrowed);
    }
    if (o == kSlotNoMass && last) {  // no residual mass after rounding: the last helper draws from p_n
      RowStat* s_part = reinterpret_cast<RowStat*>(s_buf);
      if (single_restage_row(a, b, tag, d.row, s_part))
        direct_draw<DT, VEC>(a, b, d, kModeFallbackP, row_t, s_part + static_cast<size_t>(d.row) * a.C * kWaves, xs,
                             kNoStamp);
      else
        write_timed_out(a, b, tid, kThreads);
    }
  } else if (!ok && last) {  // the wait gave up: flag the sequence
    write_timed_out(a, b, tid, kThreads);
  }
  // the last helper advances the sequence's run counter once the other helpers have read it
  // (lane 0 alone: the other waves may have left); the words not seen while it waited (s_nseen
  // counts those seen, as of the wait's last barrier) are polled now
  if (last && tid == 0) {
    if (s_nseen < CP - 1)
      for (int t2 = 0; t2 + 1 < CP; ++t2) {
        uint32_t v;
        for (int polls = 0; polls < a.poll_limit && !get_tagged_u32(st + t2, tag, &v); ++polls) short_pause();
      }
    __hip_atomic_fetch_add(a.epoch + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  stamp(a, hb + kHpExit);
}

// grid = G stats workgroups, then B x CP helpers.  When B is a multiple of 8, the stats
// workgroups of XCD x (in xcd_blocked order) stream sequences [x B/8, (x+1) B/8) whole; with
// xcd_local (set for such batches) the helpers are placed so that XCD x also holds those
// sequences' helpers (helper slot h = 8 m + x serves sequence x B/8 + m / CP), so that every
// hand-over of a sequence stays on one XCD and its words go through that XCD's L2 (store_xcd;
// measured at B=64, K=5, V=128256 bf16: 41.5 -> 39.5 us per call).  (With the n-gram lookup's
// workgroups ahead of them, the finishers taking the drafts from the lookup's tagged words, the
// prompt-lookup workload ran 22.0 us per call against 20.4 for the lookup beside the separate
// stats pass: calls that draft by lookup take the separate launches.)
template <int DT, int NV, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_fused_kernel(ChainArgs a, int G, int CP) {
  // one buffer for the finisher's partials and the helpers' masses
  __shared__ __align__(16) unsigned char s_mem[kSingleMaxParts * sizeof(RowStat)];
  const int i = static_cast<int>(blockIdx.x);
  if (i < G) {
    fused_stats<DT, NV, VEC>(a, xcd_blocked(i, G), G, s_mem);
    return;
  }
  const int h = i - G;
  if (a.xcd_local) {
    const int m = h / kXcds;
    fused_helper<DT, kPoolSegments, VEC>(a, (h % kXcds) * (a.B / kXcds) + m / CP, m % CP, CP, s_mem);
  } else {
    fused_helper<DT, kPoolSegments, VEC>(a, h / CP, h % CP, CP, s_mem);
  }
}

// grid = 1: offsets and packed tokens of the batch (only when packed output is asked for).
__global__ __launch_bounds__(kThreads) void chain_pack_kernel(ChainArgs a) { chain_pack(a); }

__global__ void write_zero_offset_kernel(int32_t* offsets) {
  if (threadIdx.x == 0) offsets[0] = 0;
}

// ---------------------------------------------------------------- host side

struct ChainLayout {
  int nv, C, R, S;
  bool single;  // the shape may take the single-launch path (its regions are laid out)
  bool fused;   // the shape may take the fused path (its regions are laid out)
  int tstride, sstride;  // words per sequence of the tagged partials and of the status words
  size_t off_gath, off_part, off_wseg, off_decs, off_epoch, off_tpart, off_tprop, off_status, off_tmass, off_tdec,
      bytes;
};

// Vectors per lane in one stats chunk.  The largest chunk (16 vectors for bf16 rows read with
// 16-byte loads, else 8) that gives at least 1024 workgroups with at most kMaxChunks chunks a
// row; if none reaches 1024 workgroups within that bound (small batches), the smallest chunk
// within it but no smaller than 4 vectors (16 KiB); if even the largest chunk leaves more
// than kMaxChunks a row, the largest chunk.
// Bounding the chunks a row bounds the partials every pool task combines before it can
// decide, which sets the latency of small batches.  Measured per call: at B=64, K=5,
// V=128256 bf16, 16 vectors 50.6 us, 8 vectors 52.7, 4 vectors 58; at B=256, K=8, V=152064,
// 16 vectors 246 us, 8 vectors 269; at K=5, V=128256 bf16, B=1: 4 vectors (16 chunks) 13.1 us
// against 23.1 with 1 vector (63 chunks, the 1024-workgroup target alone), B=4: 15.9 against
// 19.0 with 2 vectors, B=16: 8 vectors 22.3 either way; at B=1, K=5, V=32000 fp32: 4 vectors
// 12.1 us, 2 vectors 12.8, 8 vectors 13.0, against 15.9 with 1 vector.  Element-wise loads keep at most 8,
// whose registers would not fit twice.  SPEC_KNOB_CHUNK_VECTORS forces 1, 2, 4 or 8, or 16
// where 16 may be chosen.
constexpr int kMaxChunks = 16;

static int chain_nv(long long rows, int V, int epv, bool vec) {
  const int forced = knob(SPEC_KNOB_CHUNK_VECTORS);
  const int top = vec && epv == 8 ? 16 : 8;
  if (forced == 16 && top == 16) return 16;
  if (forced == 1 || forced == 2 || forced == 4 || forced == 8) return forced;
  const auto chunks = [&](int nv) {
    const long long chunk = static_cast<long long>(nv) * kThreads * epv;
    return (V + chunk - 1) / chunk;
  };
  int pick = 0;
  for (int nv = top; nv >= 1; nv >>= 1) {
    if (chunks(nv) > kMaxChunks) break;  // smaller chunks only give more
    pick = nv;
    if (rows * chunks(nv) >= 1024) return nv;
  }
  return pick ? (pick < 4 ? 4 : pick) : top;
}

// `vec`: the rows can be read with 16-byte loads; `one_hot`: no draft rows (K+1 rows per
// sequence are streamed instead of 2K+1); `lookup`: the drafts come from the n-gram lookup
// (which never takes the fused launch).  They set the chunk size; the workspace regions keep
// room for 2K+1 rows either way.
static ChainLayout chain_layout(int B, int K, int V, spec_dtype_t dtype, bool vec, bool one_hot, bool prefer_single,
                                bool lookup) {
  ChainLayout L{};
  const int epv = dtype == SPEC_BF16 ? 8 : 4;
  L.R = 2 * K + 1;
  const int rows = one_hot ? K + 1 : L.R;  // rows a sequence streams
  const long long seg = static_cast<long long>(kThreads) * epv;
  const long long used = (V + seg - 1) / seg;
  L.S = static_cast<int>((used + kPoolSegments - 1) / kPoolSegments * kPoolSegments);
  const auto chunks = [&](int nv) {
    const long long chunk = static_cast<long long>(nv) * kThreads * epv;
    return static_cast<int>((V + chunk - 1) / chunk);
  };
  // the single launch: chunks of kSingleVectors vectors a lane, the whole grid (lookup and
  // (K+1) x C workgroups a sequence) within kSingleMaxGroups and a sequence's partials within
  // kSingleMaxParts
  const auto fits_single = [&](int nv) {
    const long long groups = static_cast<long long>(B) * ((K + 1) * static_cast<long long>(chunks(nv)) + 1);
    return nv == kSingleVectors && groups <= kSingleMaxGroups &&
           static_cast<long long>(rows) * chunks(nv) * kWaves <= kSingleMaxParts;
  };
  L.nv = chain_nv(static_cast<long long>(B) * rows, V, epv, vec);
  // a small batch whose chunk choice is smaller takes the single launch's chunk when that fits
  // (unless a knob forces the chunk or the separate launches)
  if (prefer_single && L.nv < kSingleVectors && knob(SPEC_KNOB_CHUNK_VECTORS) == 0 && fits_single(kSingleVectors))
    L.nv = kSingleVectors;
  // A call that takes the fused launch streams 32 KiB chunks where the rule gives 64 KiB, when
  // its partials still fit: the pass is faster with them, and with the hand-overs in one XCD's
  // L2 the doubled partials cost the finisher less than that (measured per call at B=64, K=5,
  // V=128256 bf16: 39.5 -> 38.9 us, greedy 22.4 -> 22.2 us, one-hot B=160 47.9 -> 46.0 us; the
  // separate launches keep 64 KiB chunks, B=256, K=8, V=152064: 222.8 against 225.0 us with 32 KiB)
  const long long fused_cp = one_hot ? 1 : L.S / kPoolSegments;
  if (prefer_single && !lookup && L.nv == 16 && knob(SPEC_KNOB_CHUNK_VECTORS) == 0 &&
      static_cast<long long>(rows) * chunks(8) * kWaves <= kSingleMaxParts &&
      static_cast<long long>(B) * fused_cp <= kFusedMaxHelpers)
    L.nv = 8;
  L.C = chunks(L.nv);
  const size_t segs = static_cast<size_t>(B) * L.S;
  size_t off = 256;  // bytes 0..3: the run counter
  L.off_gath = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(B) * L.R, 256);
  L.off_part = off;
  off = align_up(off + sizeof(RowStat) * static_cast<size_t>(B) * L.R * L.C * kWaves, 256);
  L.off_wseg = off;
  off = align_up(off + sizeof(SlotDouble) * segs, 256);
  L.off_decs = off;
  off = align_up(off + sizeof(ChainDecision) * static_cast<size_t>(B), 256);
  // the single-launch path's words, for shapes it may take (the device decides at call time)
  L.single = prefer_single && fits_single(L.nv);
  // the fused path: a sequence's partials within kSingleMaxParts and its pool tasks within the
  // status words
  const long long cp = one_hot ? 1 : L.S / kPoolSegments;
  L.fused = prefer_single && static_cast<long long>(rows) * L.C * kWaves <= kSingleMaxParts &&
            static_cast<long long>(B) * (static_cast<long long>(rows) * L.C + cp) <= 2147483647LL;
  if (L.single || L.fused) {
    // a sequence's tagged partials (rows x C chunks x kWaves, 3 words each) and its status words
    // (one per workgroup of a single launch, one per helper of a fused one)
    L.tstride = 3 * rows * L.C * kWaves;
    L.sstride = max((K + 1) * L.C, L.S / kPoolSegments);
    L.off_epoch = off;
    off = align_up(off + sizeof(uint32_t) * B, 256);
    L.off_tpart = off;
    off = align_up(off + sizeof(uint64_t) * static_cast<size_t>(B) * L.tstride, 256);
    L.off_status = off;
    off = align_up(off + sizeof(uint64_t) * static_cast<size_t>(B) * L.sstride, 256);
  }
  if (L.single) {
    L.off_tprop = off;
    off = align_up(off + sizeof(uint64_t) * static_cast<size_t>(B) * (2 * K + 1), 256);
    L.off_tmass = off;
    off = align_up(off + sizeof(SlotDouble) * static_cast<size_t>(B) * K * L.S, 256);
  }
  if (L.fused) {
    L.off_tdec = off;
    off = align_up(off + sizeof(uint64_t) * static_cast<size_t>(B) * kFusedDecisionWords, 256);
  }
  L.bytes = off;
  return L;
}

// Workspace bytes a chain call of this shape may need: the largest of the layouts it may take
// (the chunk size depends on the pointers' alignment, on whether draft rows are given and on
// whether a one-launch path is allowed; one_launch = false leaves the last out).
static size_t chain_workspace_bytes(int B, int K, int V, spec_dtype_t dtype, bool one_launch) {
  if (B <= 0 || K < 1 || K > SPEC_MAX_K || V < 1) return 0;
  size_t bytes = 0;
  for (int vec = 0; vec < 2; ++vec)
    for (int one_hot = 0; one_hot < 2; ++one_hot)
      for (int single = 0; single < (one_launch ? 2 : 1); ++single)
        for (int lookup = 0; lookup < 2; ++lookup) {
          const size_t b = chain_layout(B, K, V, dtype, vec != 0, one_hot != 0, single != 0, lookup != 0).bytes;
          bytes = b > bytes ? b : bytes;
        }
  return bytes;
}

// Pool workgroups the current device holds at once (cached per device).
static int pool_slots(const void* kernel, std::atomic<int>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int slots = dev < kMaxDevices ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (slots <= 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess) per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 1;
    slots = max(1, per_cu) * max(1, cus);
    if (dev < kMaxDevices) cache[dev].store(slots, std::memory_order_relaxed);
  }
  return slots;
}

// Generation of the next call's slot words: a process-wide counter with a random start,
// skipping 0.
static uint32_t next_generation() {
  static std::atomic<uint32_t> counter{[] {
    std::random_device rd;
    return static_cast<uint32_t>(rd()) ^
           static_cast<uint32_t>(std::chrono::steady_clock::now().time_since_epoch().count());
  }()};
  uint32_t g = counter.fetch_add(1u, std::memory_order_relaxed);
  if (g == 0u) g = counter.fetch_add(1u, std::memory_order_relaxed);
  return g;
}

// Phase timestamp buffer set by spec_chain_phase_stamps (null: none).
static std::atomic<unsigned long long*> g_stamps{nullptr};
static std::atomic<size_t> g_stamp_words{0};

// The stats pass (with the n-gram lookup in the same launch when `ng` is given), then the pool
// kernel and, when asked for, the packed output.
template <int DT, int NV, bool VEC>
static spec_status_t launch_chain(ChainArgs a, const NgramArgs* ng, hipStream_t stream) {
  a.stamps = nullptr;
  if (unsigned long long* buf = ng ? nullptr : g_stamps.load(std::memory_order_acquire)) {
    const size_t g1 = static_cast<size_t>(a.B) * a.R * a.C;
    const size_t need = 2 * g1 + kStampsPerTask * static_cast<size_t>(a.B) * (a.draft ? a.S / kPoolSegments : 1);
    if (need <= g_stamp_words.load(std::memory_order_acquire)) {
      a.stamps = buf;
      a.stamps_pool = 2 * g1;
    }
  }
  static std::atomic<int> slots_cache[kMaxDevices];
  static std::atomic<int> single_cache[2][kMaxDevices];
  if constexpr (NV == kSingleVectors) {
    if (a.tmass && knob(SPEC_KNOB_SINGLE_LAUNCH) == 0) {
      // one launch when the whole grid fits on the device at once (with its own stamp layout)
      ChainArgs as = a;
      as.stamps = nullptr;
      as.stamps_pool = 0;
      if (unsigned long long* buf = g_stamps.load(std::memory_order_acquire))
        if (kStampsPerTask * static_cast<size_t>(a.B) * (a.K + 1) * a.C <= g_stamp_words.load(std::memory_order_acquire))
          as.stamps = buf;
      using Kernel = void (*)(ChainArgs, NgramArgs, int);
      const Kernel kernel = a.draft ? chain_single_kernel<DT, NV, VEC, true> : chain_single_kernel<DT, NV, VEC, false>;
      const int P = ng ? a.B : 0;
      const long long total = P + static_cast<long long>(a.B) * (a.K + 1) * a.C;
      // each sequence on one XCD (see chain_single_kernel) once every XCD has a sequence: an eighth
      // of the slots for each XCD's share.  (Fewer sequences would leave XCDs idle and stream each
      // sequence's rows through one: B=1, K=5, V=32000 fp32 9.7 -> 10.7 us per call; with 8 or more,
      // B=16 one-hot, V=32000 bf16 10.5 -> 9.6 us, B=8 11.9 -> 11.7 us.)
      const long long share = static_cast<long long>((a.B + kXcds - 1) / kXcds) * ((ng ? 1 : 0) + (a.K + 1) * a.C);
      const int slots = pool_slots(reinterpret_cast<const void*>(kernel), single_cache[a.draft ? 1 : 0]);
      as.xcd_local = knob(SPEC_KNOB_XCD_LOCAL) != 0 && a.B >= kXcds && share <= slots / kXcds;
      if (total <= slots) {
        const NgramArgs none{};
        const long long grid = as.xcd_local ? kXcds * share : total;
        LaunchScope scope("chain_single", stream);
        scope.launch(kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), stream, as, ng ? *ng : none, P);
        const spec_status_t st = scope.finish();
        if (st != SPEC_OK || !a.out_packed) return st;
        LaunchScope pack("chain_pack", stream);
        pack.launch(chain_pack_kernel, dim3(1), dim3(kThreads), stream, a);
        return pack.finish();
      }
    }
  }
  if (a.tdec && !ng && knob(SPEC_KNOB_SINGLE_LAUNCH) == 0 &&
      static_cast<long long>(a.B) * (a.draft ? a.S / kPoolSegments : 1) <= kFusedMaxHelpers) {
    // the pass and the draws in one launch: G stats workgroups, then CP helpers a sequence
    const int G = a.B * a.R * a.C;
    const int CP = a.draft ? a.S / kPoolSegments : 1;
    ChainArgs af = a;  // with the fused launch's own stamp layout
    af.stamps = nullptr;
    af.stamps_pool = 0;
    if (unsigned long long* buf = g_stamps.load(std::memory_order_acquire))
      if (2 * static_cast<size_t>(G) + kFinisherStamps * static_cast<size_t>(a.B) +
              kHelperStamps * static_cast<size_t>(a.B) * CP <= g_stamp_words.load(std::memory_order_acquire))
        af.stamps = buf;
    // each sequence's workgroups on one XCD (see chain_fused_kernel): its hand-overs through that
    // XCD's L2, unless switched off
    af.xcd_local = a.B % kXcds == 0 && knob(SPEC_KNOB_XCD_LOCAL) != 0;
    LaunchScope scope("chain_fused", stream);
    scope.launch(chain_fused_kernel<DT, NV, VEC>, dim3(static_cast<unsigned>(G + a.B * CP)), dim3(kThreads), stream, af,
                 G, CP);
    const spec_status_t st = scope.finish();
    if (st != SPEC_OK || !a.out_packed) return st;
    LaunchScope pack("chain_pack", stream);
    pack.launch(chain_pack_kernel, dim3(1), dim3(kThreads), stream, a);
    return pack.finish();
  }
  {
    const long long g1 = static_cast<long long>(a.B) * a.R * a.C;
    if (ng) {
      LaunchScope scope("ngram_chain_stats", stream);
      scope.launch((ngram_chain_stats_kernel<DT, NV, VEC>), dim3(static_cast<unsigned>(a.B + g1)), dim3(kThreads),
                   stream, a, *ng);
      const spec_status_t st = scope.finish();
      if (st != SPEC_OK) return st;
    } else {
      LaunchScope scope("chain_stats", stream);
      scope.launch((chain_stats_kernel<DT, NV, VEC>), dim3(static_cast<unsigned>(g1)), dim3(kThreads), stream, a);
      const spec_status_t st = scope.finish();
      if (st != SPEC_OK) return st;
    }
  }
  {
    const auto kernel = chain_pool_kernel<DT, kPoolSegments, VEC>;
    const int CP = a.draft ? a.S / kPoolSegments : 1;  // tasks per sequence
    // More pool tasks than fit at once: one decision a sequence beforehand, which the tasks read
    // (measured at B=256, K=8, V=152064: pool 43.1 -> 33.7 us plus 4.2 for the decisions, 230.0 ->
    // 225.3 us per call; at B=64, K=5, V=128256, whose 1024 tasks all fit, 12.8 -> 11.7 plus 4.2)
    if (a.draft && a.decs &&
        static_cast<long long>(a.B) * CP > pool_slots(reinterpret_cast<const void*>(kernel), slots_cache)) {
      LaunchScope scope("chain_decide", stream);
      scope.launch(chain_decide_kernel<DT>, dim3(static_cast<unsigned>(a.B)), dim3(kThreads), stream, a);
      const spec_status_t st = scope.finish();
      if (st != SPEC_OK) return st;
      a.decided = 1;
    }
    // one waiting task per sequence: at most half as many sequences per launch as fit at once
    const int per_launch = max(1, pool_slots(reinterpret_cast<const void*>(kernel), slots_cache) / 2);
    a.xcd_local = knob(SPEC_KNOB_XCD_LOCAL) != 0;  // (used by launches of a multiple of 8 sequences)
    for (int b0 = 0; b0 < a.B; b0 += per_launch) {
      const int bs = min(per_launch, a.B - b0);
      LaunchScope scope("chain_pool", stream);
      scope.launch(kernel, dim3(static_cast<unsigned>(static_cast<long long>(bs) * CP)), dim3(kThreads), stream, a, b0,
                   CP);
      const spec_status_t st = scope.finish();
      if (st != SPEC_OK) return st;
    }
  }
  if (!a.out_packed) return SPEC_OK;
  LaunchScope scope("chain_pack", stream);
  scope.launch(chain_pack_kernel, dim3(1), dim3(kThreads), stream, a);
  return scope.finish();
}

template <int DT>
static spec_status_t dispatch_chain(int nv, bool vec, const ChainArgs& a, const NgramArgs* ng, hipStream_t s) {
  switch (nv) {
    case 16:  // chosen only for bf16 rows with 16-byte loads
      if constexpr (DT == kBF16) {
        if (vec) return launch_chain<DT, 16, true>(a, ng, s);
      }
      return fail(SPEC_ERR_UNSUPPORTED, "16-vector chunks need bf16 rows and 16-byte loads");
    case 8: return vec ? launch_chain<DT, 8, true>(a, ng, s) : launch_chain<DT, 8, false>(a, ng, s);
    case 4: return vec ? launch_chain<DT, 4, true>(a, ng, s) : launch_chain<DT, 4, false>(a, ng, s);
    case 2: return vec ? launch_chain<DT, 2, true>(a, ng, s) : launch_chain<DT, 2, false>(a, ng, s);
    default: return vec ? launch_chain<DT, 1, true>(a, ng, s) : launch_chain<DT, 1, false>(a, ng, s);
  }
}

// ---------------------------------------------------------------- allocation-free variant
//
// spec_verify_chain_noalloc runs spec_verify_chain on this file-scope device array instead of
// a caller's workspace.  Each device the library runs on holds its own copy until the process
// ends.  Host code never passes the array's name to a kernel (on the host it only stands in
// for the symbol): the device address comes from hipGetSymbolAddress, taken once per device
// on that device's first call and kept.  Nothing in the array needs to start at zero: the
// values the kernels hand each other carry the call's generation number, and the run
// counter at its start may hold anything.
constexpr size_t kScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first call there).
static spec_status_t scratch_address(void** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPEC_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SPEC_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess || !p)
      return fail(SPEC_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(g));
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SPEC_OK;
}

}  // namespace specv

using namespace specv;

extern "C" {

size_t spec_verify_chain_workspace_size(int B, int K, int V, spec_dtype_t dtype) {
  return chain_workspace_bytes(B, K, V, dtype, true);
}

}  // extern "C"

// spec_verify_chain, and (with ng) the n-gram lookup's fused form: draft_tokens and draft_len
// are then the lookup's outputs, written by the first launch.
static spec_status_t verify_chain_impl(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                       const int32_t* draft_tokens, const int32_t* draft_len,
                                       const float* temperature, const float* u_accept, const float* u_final,
                                       int B, int K, int V,
                                       int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                       int32_t* out_packed, int32_t* out_offsets,
                                       void* workspace, size_t workspace_bytes, const NgramArgs* ng,
                                       bool one_launch, spec_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return fail(SPEC_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || K < 1 || V < 1) return fail(SPEC_ERR_INVALID_ARG, "need B >= 0, K >= 1, V >= 1 (got %d, %d, %d)", B, K, V);
  if (K > SPEC_MAX_K) return fail(SPEC_ERR_UNSUPPORTED, "K = %d exceeds SPEC_MAX_K = %d", K, SPEC_MAX_K);
  if ((out_packed == nullptr) != (out_offsets == nullptr))
    return fail(SPEC_ERR_INVALID_ARG, "out_packed and out_offsets must both be given or both be NULL");
  if (B == 0) {
    if (out_offsets) {
      LaunchScope scope("chain_empty", s);
      scope.launch(write_zero_offset_kernel, dim3(1), dim3(64), s, out_offsets);
      return scope.finish();
    }
    return SPEC_OK;
  }
  if (!target_logits || !draft_tokens || !temperature || !u_accept || !u_final || !out_tokens || !out_num_accepted)
    return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  const int esize = dtype == SPEC_BF16 ? 2 : 4;
  if (static_cast<double>(B) * (K + 1) * V >= 140737488355328.0)
    return fail(SPEC_ERR_UNSUPPORTED, "B*(K+1)*V too large");
  const bool vec = (static_cast<size_t>(V) * esize) % 16 == 0 && aligned16(target_logits) &&
                   (draft_logits == nullptr || aligned16(draft_logits));
  const ChainLayout L =
      chain_layout(B, K, V, dtype, vec, draft_logits == nullptr, one_launch && knob(SPEC_KNOB_SINGLE_LAUNCH) == 0,
                   ng != nullptr);
  const double groups = static_cast<double>(B) * L.R * L.C;
  if (groups > 2147483647.0) return fail(SPEC_ERR_UNSUPPORTED, "grid of %.0f workgroups too large", groups);
  if (L.S > 4 * kThreads)
    return fail(SPEC_ERR_UNSUPPORTED, "V = %d is too large (at most %d segments of %d elements)", V, 4 * kThreads,
                kThreads * (dtype == SPEC_BF16 ? 8 : 4));
  if (!workspace) return fail(SPEC_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(SPEC_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (workspace_bytes < L.bytes)
    return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.bytes);

  ChainArgs a{};
  a.target = target_logits;
  a.draft = draft_logits;
  a.tokens = draft_tokens;
  a.draft_len = draft_len;
  a.temperature = temperature;
  a.u_accept = u_accept;
  a.u_final = u_final;
  a.B = B;
  a.K = K;
  a.V = V;
  a.C = L.C;
  a.nv = L.nv;
  a.S = L.S;
  a.R = draft_logits ? L.R : K + 1;  // the workspace is laid out for 2K+1 rows; fewer fit
  a.out_tokens = out_tokens;
  a.out_num = out_num_accepted;
  a.out_probs = out_probs;
  a.out_packed = out_packed;
  a.out_offsets = out_offsets;
  char* ws = static_cast<char*>(workspace);
  a.gen = next_generation();
  a.poll_limit = knob(SPEC_KNOB_POLL_LIMIT);
  a.stats_copy = ng ? 0 : 1;
  a.runs = static_cast<uint32_t*>(workspace);
  a.gath = reinterpret_cast<float*>(ws + L.off_gath);
  a.part = reinterpret_cast<RowStat*>(ws + L.off_part);
  a.wseg = reinterpret_cast<SlotDouble*>(ws + L.off_wseg);
  a.decs = reinterpret_cast<ChainDecision*>(ws + L.off_decs);
  a.decided = 0;
  a.xcd_local = 0;
  if (L.single || L.fused) {
    a.epoch = reinterpret_cast<uint32_t*>(ws + L.off_epoch);
    a.tpart = reinterpret_cast<uint64_t*>(ws + L.off_tpart);
    a.status = reinterpret_cast<uint64_t*>(ws + L.off_status);
    a.tstride = L.tstride;
    a.sstride = L.sstride;
  }
  if (L.single) {
    a.tprop = reinterpret_cast<uint64_t*>(ws + L.off_tprop);
    a.tmass = reinterpret_cast<SlotDouble*>(ws + L.off_tmass);
  }
  if (L.fused) a.tdec = reinterpret_cast<uint64_t*>(ws + L.off_tdec);

  if (dtype == SPEC_BF16) return dispatch_chain<kBF16>(L.nv, vec, a, ng, s);
  return dispatch_chain<kF32>(L.nv, vec, a, ng, s);
}

extern "C" {

spec_status_t spec_verify_chain(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                const int32_t* draft_tokens, const int32_t* draft_len,
                                const float* temperature, const float* u_accept, const float* u_final,
                                int B, int K, int V,
                                int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                int32_t* out_packed, int32_t* out_offsets,
                                void* workspace, size_t workspace_bytes, spec_stream_t stream) {
  return verify_chain_impl(target_logits, draft_logits, dtype, draft_tokens, draft_len, temperature, u_accept,
                           u_final, B, K, V, out_tokens, out_num_accepted, out_probs, out_packed, out_offsets,
                           workspace, workspace_bytes, nullptr, true, stream);
}

spec_status_t spec_ngram_verify(const int32_t* context, const int32_t* context_len, int L_max, int n_min, int n_max,
                                const void* target_logits, spec_dtype_t dtype, const float* temperature,
                                const float* u_accept, const float* u_final, int B, int K, int V,
                                int32_t* out_draft_tokens, int32_t* out_draft_len, int32_t* out_match_n,
                                int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                int32_t* out_packed, int32_t* out_offsets,
                                void* workspace, size_t workspace_bytes, spec_stream_t stream) {
  if (L_max < 1 || n_min < 1 || n_max < n_min)
    return fail(SPEC_ERR_INVALID_ARG, "need L_max >= 1, 1 <= n_min <= n_max");
  if (n_max > SPEC_MAX_NGRAM_N) return fail(SPEC_ERR_UNSUPPORTED, "n_max = %d exceeds SPEC_MAX_NGRAM_N", n_max);
  if (B > 0 && (!context || !context_len || !out_draft_tokens || !out_draft_len))
    return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  const NgramArgs ng{context, context_len, L_max, n_min, n_max, out_match_n};
  return verify_chain_impl(target_logits, nullptr, dtype, out_draft_tokens, out_draft_len, temperature, u_accept,
                           u_final, B, K, V, out_tokens, out_num_accepted, out_probs, out_packed, out_offsets,
                           workspace, workspace_bytes, &ng, true, stream);
}

spec_status_t spec_chain_phase_stamps(unsigned long long* buffer, size_t words) {
  g_stamp_words.store(buffer ? words : 0, std::memory_order_release);
  g_stamps.store(buffer, std::memory_order_release);
  return SPEC_OK;
}

spec_status_t spec_verify_chain_noalloc(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                        const int32_t* draft_tokens, const int32_t* draft_len,
                                        const float* temperature, const float* u_accept, const float* u_final,
                                        int B, int K, int V,
                                        int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                        int32_t* out_packed, int32_t* out_offsets, spec_stream_t stream) {
  // the one-launch paths where their hand-over words fit the scratch too, else the separate launches
  const bool one_launch = chain_workspace_bytes(B, K, V, dtype, true) <= kScratchBytes;
  const size_t need = chain_workspace_bytes(B, K, V, dtype, false);
  if (need > kScratchBytes)
    return fail(SPEC_ERR_UNSUPPORTED,
                "B = %d, K = %d, V = %d needs %zu bytes of scratch; the allocation-free call holds %zu", B, K, V, need,
                kScratchBytes);
  void* ws = nullptr;
  const spec_status_t st = scratch_address(&ws);
  if (st != SPEC_OK) return st;
  return verify_chain_impl(target_logits, draft_logits, dtype, draft_tokens, draft_len, temperature, u_accept,
                           u_final, B, K, V, out_tokens, out_num_accepted, out_probs, out_packed, out_offsets, ws,
                           kScratchBytes, nullptr, one_launch, stream);
}

}  // extern "C"
