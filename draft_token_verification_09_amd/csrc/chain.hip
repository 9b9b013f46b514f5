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
// Three kernels, streaming the vocabulary in 16-byte vectors.  No state survives a
// call: every workspace byte a kernel reads was written earlier in the same call.
//
//  chain_stats    grid = B x R x C workgroups, R = K+1 target rows (+ K draft rows),
//                 C chunks per row.  Each workgroup reduces one chunk to
//                 (o, s) = (max(l) * log2(e)/T, sum exp2(l * log2(e)/T - o)).
//  chain_decide   grid = B x C (draft logits) or B x 1 (one-hot draft).  Every
//                 workgroup of a sequence combines the chunk partials into per-row
//                 (O, S), evaluates p(x_k), q(x_k), alpha_k and the accept tests of
//                 all drafted positions at once (one lane per position) and takes
//                 the first rejection n with a wave ballot; the workgroup of chunk 0
//                 stores the decision, the accepted prefix and the probabilities.
//                 After a rejection with a draft distribution, workgroup c computes
//                 the residual mass max(0, p_n - q_n) of chunk c of row n.
//  chain_draw     grid = B.  Selects the chunk holding u * W from the chunk prefix
//                 sums (residual masses, or, for a bonus draw from p and for a
//                 one-hot draft whose residual is p without x_n, masses that follow
//                 from chain_stats' partials), re-reads that one chunk, finds the
//                 token in vocabulary order and writes the outputs.
//
// Softmax is evaluated in the exp2 domain: with scale = log2(e)/T,
// p_i = exp2(l_i * scale - O) / S, where O is the float max(l) * scale used by
// every term and S = sum_chunks s_c * exp2(o_c - O).  Per-element work is fp32;
// cross-lane, cross-chunk and prefix sums are fp64.
#include <math.h>

#include "device_common.h"
#include "host_runtime.h"
#include "spec_verify.h"

namespace specv {

enum ChainMode : int { kModeInvalid = 0, kModeResidual = 1, kModeBonus = 2, kModeOneHot = 3, kModeFallbackP = 4 };

struct RowStat {
  float o;     // offset in the log2 domain: max(l) * scale over the chunk (-inf if empty)
  float pad;
  double s;    // sum over the chunk of exp2(l * scale - o)
};

struct ChainDecision {
  int mode;
  int n;         // accepted drafts
  int kb;        // draft length
  int excl_tok;  // one-hot mode: token removed from the residual
  int row;       // row (position) of the final draw
  float scale;   // log2(e) / T
  float Ot, Od;  // row offsets (target, draft)
  float invSt, invSd;
  float p_excl;  // one-hot mode: p_n(x_n)
  float pad;
  double St, Sd;
};

struct ChainArgs {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* draft_len;
  const float* temperature;
  const float* u_accept;
  const float* u_final;
  int B, K, V, C, R;
  int32_t* out_tokens;
  int32_t* out_num;
  float* out_probs;
  int32_t* out_packed;
  int32_t* out_offsets;
  RowStat* part;
  ChainDecision* dec;
  double* wmass;
};

template <int DT>
__device__ inline const void* target_row(const ChainArgs& a, int b, int k) {
  return static_cast<const char*>(a.target) +
         (static_cast<size_t>(b) * (a.K + 1) + k) * static_cast<size_t>(a.V) * Elem<DT>::kBytes;
}

template <int DT>
__device__ inline const void* draft_row(const ChainArgs& a, int b, int k) {
  return static_cast<const char*>(a.draft) +
         (static_cast<size_t>(b) * a.K + k) * static_cast<size_t>(a.V) * Elem<DT>::kBytes;
}

// Draft length of sequence b clamped to [0, K] (an out-of-range value is flagged later).
__device__ inline int clamped_len(const ChainArgs& a, int b) {
  if (!a.draft_len) return a.K;
  const int v = a.draft_len[b];
  return v < 0 ? 0 : (v > a.K ? a.K : v);
}

// Row rr of the stats grid: rr <= K is target row rr, otherwise draft row rr-K-1
// (draft rows exist only when draft logits are given; then R = 2K+1, else R = K+1).
__device__ inline bool row_needed(const ChainArgs& a, int rr, int kb) {
  return rr <= a.K ? (rr <= kb) : (a.draft != nullptr && rr - (a.K + 1) < kb);
}

// ---------------------------------------------------------------- decision

template <int DT>
__device__ void chain_decide_positions(const ChainArgs& a, int b, int kb, bool write_outputs, ChainDecision* out,
                                       const float* sO, const double* sS);

// Every workgroup of sequence b calls this with all lanes; the decision lands in *out
// (shared memory) in all of them, identically (same inputs, same arithmetic, same order).
// Only the workgroup with write_outputs stores it and the decision-level outputs.
template <int DT>
__device__ void chain_decide(const ChainArgs& a, int b, int kb, bool write_outputs, ChainDecision* out) {
  __shared__ float sO[2 * SPEC_MAX_K + 1];
  __shared__ double sS[2 * SPEC_MAX_K + 1];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;

  // Per-row statistics from the chunk partials.
  for (int rr = w; rr < a.R; rr += kWaves) {
    if (!row_needed(a, rr, kb)) continue;
    const RowStat* ps = a.part + (static_cast<size_t>(b) * a.R + rr) * a.C;
    float om = -INFINITY;
    for (int c = lane; c < a.C; c += 64) om = fmaxf(om, ps[c].o);
    om = wave_max(om);
    double sum = 0.0;
    for (int c = lane; c < a.C; c += 64) {
      const RowStat st = ps[c];
      if (st.o != -INFINITY) sum += st.s * static_cast<double>(exp2_fast(st.o - om));
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      sO[rr] = om;
      sS[rr] = sum;
    }
  }
  __syncthreads();
  if (w == 0) chain_decide_positions<DT>(a, b, kb, write_outputs, out, sO, sS);
  __syncthreads();
}

template <int DT>
__device__ void chain_decide_positions(const ChainArgs& a, int b, int kb, bool write_outputs, ChainDecision* out,
                                       const float* sO, const double* sS) {
  const int lane = threadIdx.x & 63;
  // One lane per drafted position: p(x_k), q(x_k), alpha_k and the accept test.
  const float T = a.temperature[b];
  const float scale = kLog2e / T;
  const int k = lane;
  const bool active = k < kb;
  bool bad = false, accepted = true;
  float P = 0.f, Q = 0.f, alpha = 0.f;
  int x = 0;
  if (active) {
    x = a.tokens[static_cast<size_t>(b) * a.K + k];
    const float u = a.u_accept[static_cast<size_t>(b) * a.K + k];
    if (x < 0 || x >= a.V || !(u > 0.f && u <= 1.f)) {
      bad = true;
    } else {
      const float lt = Elem<DT>::value(target_row<DT>(a, b, k), x);
      P = static_cast<float>(static_cast<double>(exp2_fast(fmaf(lt, scale, -sO[k]))) / sS[k]);
      if (a.draft) {
        const int rd = a.K + 1 + k;
        const float ld = Elem<DT>::value(draft_row<DT>(a, b, k), x);
        Q = static_cast<float>(static_cast<double>(exp2_fast(fmaf(ld, scale, -sO[rd]))) / sS[rd]);
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
  const int kb_raw = a.draft_len ? a.draft_len[b] : a.K;
  const float uf = a.u_final[b];
  const bool invalid = badm != 0ull || !(T > 0.f) || !(T <= 3.4e38f) || kb_raw < 0 || kb_raw > a.K ||
                       !(uf > 0.f && uf <= 1.f);
  const float Pn = __shfl(P, n < 64 ? n : 0, 64);
  const int xn = __shfl(x, n < 64 ? n : 0, 64);

  if (write_outputs && a.out_probs && k < a.K) {
    float* pr = a.out_probs + (static_cast<size_t>(b) * a.K + k) * 3;
    const bool keep = active && !invalid;
    pr[0] = keep ? P : 0.f;
    pr[1] = keep ? Q : 0.f;
    pr[2] = keep ? alpha : 0.f;
  }
  int32_t* ot = a.out_tokens + static_cast<size_t>(b) * (a.K + 1);
  if (write_outputs) {
    if (invalid) {
      for (int kk = lane; kk <= a.K; kk += 64) ot[kk] = -1;
    } else if (k < n) {
      ot[k] = x;
    }
  }
  if (lane == 0) {
    if (write_outputs) a.out_num[b] = invalid ? -1 : n;
    ChainDecision d{};
    d.n = n;
    d.kb = kb;
    d.scale = scale;
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
      d.invSd = static_cast<float>(1.0 / d.Sd);
    } else {
      d.mode = kModeOneHot;
      d.row = n;
      d.excl_tok = xn;
      d.p_excl = Pn;
    }
    if (!invalid) {
      d.Ot = sO[d.row];
      d.St = sS[d.row];
      d.invSt = static_cast<float>(1.0 / d.St);
    }
    *out = d;
    if (write_outputs) a.dec[b] = d;
  }
}

template <int DT, int NV, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_stats_kernel(ChainArgs a) {
  __shared__ float s_f[kWaves];
  __shared__ double s_d[kWaves];
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  const int g = blockIdx.x;
  const int c = g % a.C;
  const int rr = (g / a.C) % a.R;
  const int b = g / (a.C * a.R);
  const int kb = clamped_len(a, b);
  if (!row_needed(a, rr, kb)) return;
  const void* row = rr <= a.K ? target_row<DT>(a, b, rr) : draft_row<DT>(a, b, rr - (a.K + 1));
  const float scale = kLog2e / a.temperature[b];

  u32x4 raw[NV];
  load_chunk<DT, NV, VEC>(raw, row, a.V, c);
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int i = 0; i < E; ++i) m = fmaxf(m, EL::get(raw[j], i));
  float o = -INFINITY, s = 0.f;
  if (m != -INFINITY) {
    o = m * scale;
    float acc[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      acc[j] = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[j] += exp2_fast(fmaf(EL::get(raw[j], i), scale, -o));
    }
#pragma unroll
    for (int h = NV / 2; h >= 1; h >>= 1)
#pragma unroll
      for (int j = 0; j < h; ++j) acc[j] += acc[j + h];
    s = acc[0];
  }
  const float ob = block_max(o, s_f);
  const double contrib = (o == -INFINITY) ? 0.0 : static_cast<double>(s) * static_cast<double>(exp2_fast(o - ob));
  const double sb = block_sum(contrib, s_d);
  if (threadIdx.x == 0) a.part[(static_cast<size_t>(b) * a.R + rr) * a.C + c] = RowStat{ob, 0.f, sb};
}

// ---------------------------------------------------------------- final draw (one workgroup per sequence)

// Weight of element e of the final draw's row(s) for a chunk already in registers.
template <int DT>
__device__ inline float draw_weight(int mode, const ChainDecision& d, float lt, float ld, int e) {
  const float p = exp2_fast(fmaf(lt, d.scale, -d.Ot)) * d.invSt;
  if (mode == kModeResidual) {
    const float q = exp2_fast(fmaf(ld, d.scale, -d.Od)) * d.invSd;
    return fmaxf(0.f, p - q);
  }
  if (mode == kModeOneHot && e == d.excl_tok) return 0.f;
  return p;
}

template <int DT, int NV, bool VEC>
__device__ void chain_finalize(const ChainArgs& a, int b, ChainDecision d) {
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  constexpr int kChunk = ChunkShape<DT, NV>::kChunk;
  __shared__ double s_d[kWaves];
  __shared__ int s_i[kWaves];
  __shared__ double s_seg[NV][kWaves];
  __shared__ double s_base;
  __shared__ int s_c;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int C = a.C;

  if (d.mode != kModeInvalid) {
    int mode = d.mode;
    const float uf = a.u_final[b];
    const int per = (C + kThreads - 1) / kThreads;
    const int c0 = tid * per;
    const int c1 = min(C, c0 + per);

    auto chunk_mass = [&](int c) -> double {
      if (mode == kModeResidual) return a.wmass[static_cast<size_t>(b) * C + c];
      const RowStat st = a.part[(static_cast<size_t>(b) * a.R + d.row) * C + c];
      double mc = st.o == -INFINITY ? 0.0 : st.s * static_cast<double>(exp2_fast(st.o - d.Ot)) / d.St;
      if (mode == kModeOneHot && c == d.excl_tok / kChunk) mc = fmax(0.0, mc - static_cast<double>(d.p_excl));
      return mc;
    };

    // Chunk prefix sums (fp64, chunk order); W = their total.
    double local = 0.0;
    for (int c = c0; c < c1; ++c) local += chunk_mass(c);
    double W = block_sum(local, s_d);
    if (!(W > 0.0) && mode == kModeResidual) {
      mode = kModeFallbackP;  // residual lost to rounding: draw from p_n itself
      local = 0.0;
      for (int c = c0; c < c1; ++c) local += chunk_mass(c);
      W = block_sum(local, s_d);
    }
    const double t = static_cast<double>(uf) * W;
    // exclusive prefix of this lane's chunk range
    const double incl = wave_inclusive_scan(local);
    __syncthreads();
    if (lane == 63) s_d[w] = incl;
    __syncthreads();
    double before = incl - local;
    for (int i = 0; i < w; ++i) before += s_d[i];
    int cand = INT_MAX;
    {
      double run = before;
      for (int c = c0; c < c1; ++c) {
        const double mc = chunk_mass(c);
        run += mc;
        if (run >= t && mc > 0.0) {
          cand = c;
          break;
        }
      }
    }
    int csel = block_min_int(cand, s_i);
    if (csel == INT_MAX) {  // rounding left t above every prefix: last chunk with mass
      int lastc = -1;
      for (int c = c0; c < c1; ++c)
        if (chunk_mass(c) > 0.0) lastc = c;
      csel = block_max_int(lastc, s_i);
      if (csel < 0) csel = 0;
    }
    if (c0 <= csel && csel < c1) {
      double run = before;
      for (int c = c0; c < csel; ++c) run += chunk_mass(c);
      s_base = run;
    }
    __syncthreads();
    const double t_loc = t - s_base;

    // Re-read the selected chunk.  Vocabulary order inside a chunk is segment-major,
    // then lane, then element: each lane sums its vector of every segment, a block
    // scan of those sums finds the (segment, lane) whose range reaches t_loc, and
    // that one lane scans its own vector element by element.
    const int base = csel * kChunk;
    const void* row_t = target_row<DT>(a, b, d.row);
    const void* row_d = mode == kModeResidual ? draft_row<DT>(a, b, d.row) : nullptr;
    float seg_local[NV];
    int last_pos = -1;
    {
      u32x4 rt[NV], rd[NV];
      load_chunk<DT, NV, VEC>(rt, row_t, a.V, csel);
      if (mode == kModeResidual) load_chunk<DT, NV, VEC>(rd, row_d, a.V, csel);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        float sj = 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int e = base + (j * kThreads + tid) * E + i;
          const float ld = mode == kModeResidual ? EL::get(rd[j], i) : 0.f;
          const float wv = e < a.V ? draw_weight<DT>(mode, d, EL::get(rt[j], i), ld, e) : 0.f;
          sj += wv;
          if (wv > 0.f) last_pos = e;
        }
        seg_local[j] = sj;
      }
    }
    double seg_incl[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      seg_incl[j] = wave_inclusive_scan(static_cast<double>(seg_local[j]));
      if (lane == 63) s_seg[j][w] = seg_incl[j];
    }
    __syncthreads();
    int key = INT_MAX;
    double key_before = 0.0;
    double seg_base = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      double before = seg_base + seg_incl[j] - static_cast<double>(seg_local[j]);
      for (int i = 0; i < w; ++i) before += s_seg[j][i];
      if (key == INT_MAX && seg_local[j] > 0.f && before + static_cast<double>(seg_local[j]) >= t_loc) {
        key = j * kThreads + tid;
        key_before = before;
      }
      for (int i = 0; i < kWaves; ++i) seg_base += s_seg[j][i];
    }
    const int kmin = block_min_int(key, s_i);
    int y;
    if (kmin == INT_MAX) {  // rounding left t_loc above the chunk total: last positive weight
      y = block_max_int(last_pos, s_i);
      if (y < 0) y = base;    // unreachable: the selected chunk has positive mass
    } else {
      if (key == kmin) {
        const int e0 = base + kmin * E;
        const u32x4 vt = load_vector<DT, VEC>(row_t, a.V, e0);
        u32x4 vd = vt;
        if (mode == kModeResidual) vd = load_vector<DT, VEC>(row_d, a.V, e0);
        double run = key_before;
        int pick = -1, lastp = -1;
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int e = e0 + i;
          const float ld = mode == kModeResidual ? EL::get(vd, i) : 0.f;
          const float wv = e < a.V ? draw_weight<DT>(mode, d, EL::get(vt, i), ld, e) : 0.f;
          run += wv;
          if (wv > 0.f) {
            lastp = e;
            if (pick < 0 && run >= t_loc) pick = e;
          }
        }
        s_c = pick >= 0 ? pick : lastp;
      }
      __syncthreads();
      y = s_c;
    }

    const int n = d.n;
    int32_t* ot = a.out_tokens + static_cast<size_t>(b) * (a.K + 1);
    for (int kk = n + tid; kk <= a.K; kk += kThreads) ot[kk] = (kk == n) ? y : -1;

    if (a.out_packed) {
      double cnt = 0.0;
      for (int bb = tid; bb < b; bb += kThreads) {
        const ChainDecision e = a.dec[bb];
        cnt += e.mode == kModeInvalid ? 0.0 : static_cast<double>(e.n + 1);
      }
      const int off = static_cast<int>(block_sum(cnt, s_d));
      for (int i = tid; i <= n; i += kThreads)
        a.out_packed[off + i] = i < n ? a.tokens[static_cast<size_t>(b) * a.K + i] : y;
      if (tid == 0) {
        a.out_offsets[b] = off;
        if (b == a.B - 1) a.out_offsets[a.B] = off + n + 1;
      }
    }
    return;
  }

  // Invalid sequence: no tokens, only its packed offset.
  if (a.out_packed) {
    double cnt = 0.0;
    for (int bb = tid; bb < b; bb += kThreads) {
      const ChainDecision e = a.dec[bb];
      cnt += e.mode == kModeInvalid ? 0.0 : static_cast<double>(e.n + 1);
    }
    const int off = static_cast<int>(block_sum(cnt, s_d));
    if (tid == 0) {
      a.out_offsets[b] = off;
      if (b == a.B - 1) a.out_offsets[a.B] = off;
    }
  }
}

// Residual mass max(0, p_n - q_n) of one chunk of a rejected sequence's row pair.
// grid = B x C2 (C2 = C with draft logits, else 1).  Every workgroup of sequence b
// evaluates the sequence's decision from chain_stats' partials; the one with c == 0
// stores it with the accepted prefix, the probabilities and the count.  With a
// rejection and a draft distribution, workgroup c then computes the residual mass
// max(0, p_n - q_n) of chunk c of row n.
template <int DT, int NV, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_decide_kernel(ChainArgs a, int C2) {
  __shared__ double s_d[kWaves];
  __shared__ ChainDecision s_dec;
  using EL = Elem<DT>;
  constexpr int E = EL::kPerVec;
  const int g = blockIdx.x;
  const int c = g % C2;
  const int b = g / C2;
  chain_decide<DT>(a, b, clamped_len(a, b), c == 0, &s_dec);
  const ChainDecision d = s_dec;
  if (d.mode != kModeResidual) return;
  u32x4 rt[NV], rd[NV];
  load_chunk<DT, NV, VEC>(rt, target_row<DT>(a, b, d.row), a.V, c);
  load_chunk<DT, NV, VEC>(rd, draft_row<DT>(a, b, d.row), a.V, c);
  float acc[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    acc[j] = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float p = exp2_fast(fmaf(EL::get(rt[j], i), d.scale, -d.Ot)) * d.invSt;
      const float q = exp2_fast(fmaf(EL::get(rd[j], i), d.scale, -d.Od)) * d.invSd;
      acc[j] += fmaxf(0.f, p - q);
    }
  }
#pragma unroll
  for (int h = NV / 2; h >= 1; h >>= 1)
#pragma unroll
    for (int j = 0; j < h; ++j) acc[j] += acc[j + h];
  const double sb = block_sum(static_cast<double>(acc[0]), s_d);
  if (threadIdx.x == 0) a.wmass[static_cast<size_t>(b) * a.C + c] = sb;
}

// The final draw of each sequence (one workgroup per sequence).
template <int DT, int NV, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_draw_kernel(ChainArgs a) {
  const int b = blockIdx.x;
  chain_finalize<DT, NV, VEC>(a, b, a.dec[b]);
}

__global__ void write_zero_offset_kernel(int32_t* offsets) {
  if (threadIdx.x == 0) offsets[0] = 0;
}

// ---------------------------------------------------------------- host side

struct ChainLayout {
  int nv, C, R;
  size_t off_part, off_dec, off_wmass, bytes;
};

static ChainLayout chain_layout(int B, int K, int V, spec_dtype_t dtype) {
  ChainLayout L{};
  const int epv = dtype == SPEC_BF16 ? 8 : 4;
  L.R = 2 * K + 1;
  L.nv = choose_nv(static_cast<long long>(B) * L.R, V, epv, 1024);
  const long long chunk = static_cast<long long>(L.nv) * kThreads * epv;
  L.C = static_cast<int>((V + chunk - 1) / chunk);
  size_t off = 0;
  L.off_part = off;
  off = align_up(off + sizeof(RowStat) * static_cast<size_t>(B) * L.R * L.C, 256);
  L.off_dec = off;
  off = align_up(off + sizeof(ChainDecision) * static_cast<size_t>(B), 256);
  L.off_wmass = off;
  off = align_up(off + sizeof(double) * static_cast<size_t>(B) * L.C, 256);
  L.bytes = off;
  return L;
}

template <int DT, int NV, bool VEC>
static spec_status_t launch_chain(const ChainArgs& a, hipStream_t stream) {
  {
    const long long g1 = static_cast<long long>(a.B) * a.R * a.C;
    LaunchScope scope("chain_stats", stream);
    hipLaunchKernelGGL((chain_stats_kernel<DT, NV, VEC>), dim3(static_cast<unsigned>(g1)), dim3(kThreads), 0, stream, a);
    const spec_status_t st = scope.finish();
    if (st != SPEC_OK) return st;
  }
  {
    const int C2 = a.draft ? a.C : 1;  // a one-hot draft never takes the residual path
    const long long g2 = static_cast<long long>(a.B) * C2;
    LaunchScope scope("chain_decide", stream);
    hipLaunchKernelGGL((chain_decide_kernel<DT, NV, VEC>), dim3(static_cast<unsigned>(g2)), dim3(kThreads), 0, stream,
                       a, C2);
    const spec_status_t st = scope.finish();
    if (st != SPEC_OK) return st;
  }
  LaunchScope scope("chain_draw", stream);
  hipLaunchKernelGGL((chain_draw_kernel<DT, NV, VEC>), dim3(static_cast<unsigned>(a.B)), dim3(kThreads), 0, stream, a);
  return scope.finish();
}

template <int DT>
static spec_status_t dispatch_chain(int nv, bool vec, const ChainArgs& a, hipStream_t s) {
  switch (nv) {
    case 8: return vec ? launch_chain<DT, 8, true>(a, s) : launch_chain<DT, 8, false>(a, s);
    case 4: return vec ? launch_chain<DT, 4, true>(a, s) : launch_chain<DT, 4, false>(a, s);
    case 2: return vec ? launch_chain<DT, 2, true>(a, s) : launch_chain<DT, 2, false>(a, s);
    default: return vec ? launch_chain<DT, 1, true>(a, s) : launch_chain<DT, 1, false>(a, s);
  }
}

}  // namespace specv

using namespace specv;

extern "C" {

size_t spec_verify_chain_workspace_size(int B, int K, int V, spec_dtype_t dtype) {
  if (B <= 0 || K < 1 || K > SPEC_MAX_K || V < 1) return 0;
  return chain_layout(B, K, V, dtype).bytes;
}

spec_status_t spec_verify_chain(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                const int32_t* draft_tokens, const int32_t* draft_len,
                                const float* temperature, const float* u_accept, const float* u_final,
                                int B, int K, int V,
                                int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                int32_t* out_packed, int32_t* out_offsets,
                                void* workspace, size_t workspace_bytes, spec_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return fail(SPEC_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || K < 1 || V < 1) return fail(SPEC_ERR_INVALID_ARG, "need B >= 0, K >= 1, V >= 1 (got %d, %d, %d)", B, K, V);
  if (K > SPEC_MAX_K) return fail(SPEC_ERR_UNSUPPORTED, "K = %d exceeds SPEC_MAX_K = %d", K, SPEC_MAX_K);
  if ((out_packed == nullptr) != (out_offsets == nullptr))
    return fail(SPEC_ERR_INVALID_ARG, "out_packed and out_offsets must both be given or both be NULL");
  if (B == 0) {
    if (out_offsets) {
      LaunchScope scope("chain_empty", s);
      hipLaunchKernelGGL(write_zero_offset_kernel, dim3(1), dim3(64), 0, s, out_offsets);
      return scope.finish();
    }
    return SPEC_OK;
  }
  if (!target_logits || !draft_tokens || !temperature || !u_accept || !u_final || !out_tokens || !out_num_accepted)
    return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  const int esize = dtype == SPEC_BF16 ? 2 : 4;
  if (static_cast<double>(B) * (K + 1) * V >= 140737488355328.0)
    return fail(SPEC_ERR_UNSUPPORTED, "B*(K+1)*V too large");
  const ChainLayout L = chain_layout(B, K, V, dtype);
  const double groups = static_cast<double>(B) * L.R * L.C;
  if (groups > 2147483647.0) return fail(SPEC_ERR_UNSUPPORTED, "grid of %.0f workgroups too large", groups);
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
  a.R = draft_logits ? L.R : K + 1;  // the workspace is laid out for 2K+1 rows; fewer fit
  a.out_tokens = out_tokens;
  a.out_num = out_num_accepted;
  a.out_probs = out_probs;
  a.out_packed = out_packed;
  a.out_offsets = out_offsets;
  char* ws = static_cast<char*>(workspace);
  a.part = reinterpret_cast<RowStat*>(ws + L.off_part);
  a.dec = reinterpret_cast<ChainDecision*>(ws + L.off_dec);
  a.wmass = reinterpret_cast<double*>(ws + L.off_wmass);

  const bool vec = (static_cast<size_t>(V) * esize) % 16 == 0 && aligned16(target_logits) &&
                   (draft_logits == nullptr || aligned16(draft_logits));
  if (dtype == SPEC_BF16) return dispatch_chain<kBF16>(L.nv, vec, a, s);
  return dispatch_chain<kF32>(L.nv, vec, a, s);
}

}  // extern "C"
