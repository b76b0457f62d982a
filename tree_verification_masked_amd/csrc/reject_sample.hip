// Tree rejection sampling with sibling fallthrough, and greedy verification.
//
// "Eagle vs DFlash" (gingerlabs.ai), "Target-model decoding is serial": a drafted
// token x is accepted with probability min(1, p(x)/q(x)); on rejection the
// replacement is drawn from norm(max(0, p - q)).  Tree-verification notes
// (zhangshuibai.github.io), "Tree Verification 详解" part C: siblings share the
// draft distribution produced at their parent; after a rejected sibling the
// rejected draft mass is removed from the parent's target distribution and the
// next sibling is tested against that residual; if all siblings fail the bonus is
// drawn from the residual at the parent; part G: at a leaf the bonus is drawn from
// the leaf's target distribution.
//
// Residual in closed form.  With q fixed, after j rejections the residual is
//   r_j = max(0, p - c_j q) / W(c_j),   W(c) = sum_x max(0, p(x) - c q(x)),
// c_0 = 0, W(0) = 1 and c_{j+1} = c_j + W(c_j) (kept at c_j when W(c_{j+1}) = 0,
// where the residual is left unchanged).  A sibling test then needs p(x), q(x) of
// one token plus the scalars (c_j, W(c_j)).
//
// Every node is evaluated in parallel (the uniforms are indexed by node and child,
// so a node's outcome does not depend on how the walk reached it); the walk from
// the root then only follows the per-node results.  One launch at T > 0, with a
// "planner" workgroup and one workgroup per 4096-token chunk for every node slot.
// Each of them derives the node's plan itself from the inputs: the row statistics
// of the node's target and draft rows (merged from the logit pass's chunk
// partials), the tree's verdict, the node's children, their tested tokens' p and q
// (fp64) and the first-child test.
//   planner  a leaf draws its bonus from p (the chunk that holds the target is
//            found from the chunk partials and scanned); a node whose first child
//            is accepted is done; either is reported to its request here.
//   chunks   only an internal node keeps them.  Its chunk of both rows is loaded at
//            once and held in registers as exact fixed-point masses, and the sums
//            of the first threshold (c = 1, whatever the first test gives) go out
//            before the plan is known.  When the first child is rejected the
//            node's chunks follow the sibling chain level by level: after each
//            rejection every chunk sums, exactly, the masses of its tokens with
//            p - c q > 0 for the new threshold c, publishes its two sums as tagged
//            words and reads every other chunk's words of that level, so all of
//            them hold the same exact W(c) and take the same next step.  When every
//            child is rejected, the per-chunk sums locate the chunk of the terminal
//            draw and only that chunk's workgroup scans it.  The node's last chunk
//            to finish clears its words; a chain node is reported by its chunks.
// The request's last reported node walks from the root and writes the outputs.
// The workgroups of one node are placed on one XCD (the node of ordinal o, in group
// x = o mod nx, takes blockIdx = nx * i + x, which the hardware dispatches to one
// XCD), so their words pass through that XCD's L2; within a group, blocks of nodes
// put their planners ahead of their chunks, every request's first node slots first.  Vocabularies above 64 chunks spread a node over
// the whole device with device-scope words.  A planner never waits, and a node's
// chunks wait only for each other, so the waits end whenever every chunk of a node
// can be resident at once (checked on the host from the occupancy); every wait is
// bounded besides: one that gives up reports SPEC_ERR_TIMEOUT and the call still
// ends normally.
// Masses are summed as exact integers: the fp32 unnormalised mass exp((l - m)/T)
// in [0, 1] is truncated to a multiple of 2^-42 (bit arithmetic, no rounding), so
// the sums are exact, independent of summation order and bitwise reproducible;
// the normalisation 1/Z is applied once to each sum.
#include <algorithm>

#include "common.hpp"
#include "greedy_walk.hpp"

namespace spectree {

constexpr int kThreads = 512;                // threads of a workgroup (one chunk of one node)
constexpr int kPer = kChunk / kThreads;      // tokens of a row per thread
constexpr int kQuarters = kPer / 4;          // 16-byte loads of a row per thread
constexpr double kFx = 4398046511104.0;      // 2^42
constexpr double kFxInv = 1.0 / kFx;
constexpr int kTagBits = 8;                  // level tag in the low bits of a published sum
constexpr uint32_t kWaitDefault = 1u << 22;  // polls before a wait gives up
constexpr int kLocalMaxChunks = 64;          // a node's chunks fit one XCD
constexpr int kDiagLevels = 0, kDiagTimeouts = 1;

struct NodeRes {
  int32_t acc, term, err, pad;  // err: 1 invalid row, 2 a wait gave up
};
struct SampWs {                    // nd = b * n_max + n
  uint32_t* diag;                  // [4]  cumulative counters (kDiag*)
  NodeRes* res;                    // [nd] node results, read by the request's walk
  uint32_t* req_count;             // [batch] nodes reported (self-resetting)
  uint32_t* exit_count;            // [nd] chunks of a chain node finished (self-resetting)
  unsigned long long* slot;        // [nd][2][nch][2] tagged (sum P, sum Q) of a level, by level parity
};
struct RejArgs {
  const float *tgt_logits, *tgt_max;   // tgt_max: T == 0 (NaN marks an invalid row)
  const int32_t* tgt_argmax;           // T == 0
  const float *tgt_chunk_max, *dft_chunk_max;    // T > 0: chunk maxima (NaN: invalid chunk)
  const double *tgt_chunk_sum, *dft_chunk_sum;   // T > 0: chunk sums of exp((l - m_c) / T)
  const float* dft_logits;
  double inv_t, inv_td;
  ExpScale est, esd;
  const int32_t *tokens, *parent, *n_nodes;
  const float *u_accept, *u_sample;
  int32_t batch, n_max, vocab, nch;
  int32_t vec;  // rows start 16-byte aligned (vocab % 4 == 0, aligned bases)
  int32_t *accepted_child, *term_token, *status;
  int32_t *path_nodes, *out_tokens, *accept_len;  // optional: the accepted path too
};

// The request's accepted path from the walk's results in LDS (the rules of
// spec_accept_path), when the caller asked for it.  Called by the whole workgroup.
__device__ inline void emit_path(const RejArgs& a, int b, const int* s_oacc, const int* s_oterm, const int* s_tok,
                                 int nb, int* s_pn, int* s_ot, int* s_len) {
  if (!a.path_nodes) return;
  if (threadIdx.x == 0) {
    bool bad;
    *s_len = accept_walk(s_oacc, s_oterm, s_tok, nb, a.n_max, s_pn, s_ot, &bad);
    if (bad) report(a.status, SPEC_ERR_BAD_INPUT);
  }
  __syncthreads();
  const int64_t base = (int64_t)b * a.n_max;
  for (int i = threadIdx.x; i < a.n_max; i += blockDim.x) {
    a.path_nodes[base + i] = s_pn[i];
    a.out_tokens[base + i] = s_ot[i];
  }
  if (threadIdx.x == 0) a.accept_len[b] = *s_len;
}


// A thread's kPer tokens of a chunk held in registers: slot s is token
// c0 + 4 kThreads (s / 4) + 4 tid + s % 4, so each 16-byte load of a wavefront covers
// 1 KB of consecutive tokens and token order is (run s / 4, thread, s % 4).  Tokens
// past the vocabulary read as -inf (zero mass).
__device__ inline int slot_tok(int c0, int s) {
  return c0 + 4 * kThreads * (s >> 2) + 4 * (int)threadIdx.x + (s & 3);
}
__device__ inline void load_chunk(const float* row, int c0, int vocab, bool vec, float* x) {
#pragma unroll
  for (int q = 0; q < kQuarters; ++q) {
    const int t = c0 + 4 * kThreads * q + 4 * (int)threadIdx.x;
    if (vec && t + 4 <= vocab) {
      const float4 f = *reinterpret_cast<const float4*>(row + t);
      x[4 * q + 0] = f.x;
      x[4 * q + 1] = f.y;
      x[4 * q + 2] = f.z;
      x[4 * q + 3] = f.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * q + j] = t + j < vocab ? row[t + j] : -INFINITY;
    }
  }
}


// floor(pp * 2^42) of an unnormalised mass pp in [0, 1], by bit arithmetic (exact;
// zero and subnormals, all below 2^-42, give 0).  Branch-free.
__device__ inline long long fx42(float pp) {
  const uint32_t bits = __float_as_uint(pp);
  const int e = (int)(bits >> 23);  // pp >= 0
  const uint64_t m = (uint64_t)((bits & 0x7fffffu) | 0x800000u);
  const int sh = e - 108;  // pp * 2^42 = m * 2^(e - 150 + 42), sh <= 19
  const uint64_t up = m << max(sh, 0), down = m >> min(-sh, 63);
  const uint64_t v = sh >= 0 ? up : down;
  return (e == 0 || e > 127) ? 0 : (long long)v;
}


// The sibling test u < r(x) / q(x) with r = max(0, p - c q) / W, as u W q(x) <
// max(0, p(x) - c q(x)) (W > 0): q(x) == 0 accepts exactly when the residual mass is
// positive, the ratio +inf.
__device__ inline bool sibling_accepts(float u, double px, double qx, double c, double W) {
  return (double)u * (W * qx) < fmax(0.0, px - c * qx);
}


__device__ inline long long block_sum_ll(long long v, long long* s_ll) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum_ll(v);
  __syncthreads();
  if (lane == 0) s_ll[wid] = v;
  __syncthreads();
  long long t = 0;
  for (int i = 0; i < nw; ++i) t += s_ll[i];
  return t;
}
__device__ inline double block_sum_d(double v, double* s_red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum_d(v);
  __syncthreads();
  if (lane == 0) s_red[wid] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < nw; ++i) t += s_red[i];
  return t;
}
// Exclusive prefix sum over the block in thread order (fixed combination order).
__device__ inline double block_excl_scan_d(double v, double* s_w, double* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const double inc = wave_incl_scan_d(v, lane);
  __syncthreads();
  if (lane == 63) s_w[wid] = inc;
  __syncthreads();
  double before = 0.0, all = 0.0;
  for (int i = 0; i < nw; ++i) {
    if (i < wid) before += s_w[i];
    all += s_w[i];
  }
  *total = all;
  return before + inc - v;
}


// Exclusive prefix sums of kQuarters values per thread in the order (value index,
// thread): out[q] = every thread's v[q'] for q' < q, plus v[q] of the threads before
// this one (fixed combination order).  s_w holds kQuarters * waves doubles.
__device__ inline void block_excl_scan_runs(const double* v, double* out, double* s_w) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  double inc[kQuarters];
#pragma unroll
  for (int q = 0; q < kQuarters; ++q) inc[q] = wave_incl_scan_d(v[q], lane);
  __syncthreads();
  if (lane == 63)
#pragma unroll
    for (int q = 0; q < kQuarters; ++q) s_w[q * nw + wid] = inc[q];
  __syncthreads();
  double run = 0.0;  // totals of the earlier values
#pragma unroll
  for (int q = 0; q < kQuarters; ++q) {
    double before = 0.0, all = 0.0;
    for (int i = 0; i < nw; ++i) {
      if (i < wid) before += s_w[q * nw + i];
      all += s_w[q * nw + i];
    }
    out[q] = run + before + inc[q] - v[q];
    run += all;
  }
}

// Inverse-CDF search inside the chunk at c0 held by this workgroup, mass(s) the mass
// of the token in slot s: the smallest token whose running sum added to `pre`
// exceeds `target`; the largest token with positive mass when rounding leaves no
// crossing; -1 when every mass is zero.  Called by the whole workgroup.
template <typename Mass>
__device__ int regs_scan(Mass mass, int c0, double pre, double target, double* s_w, int* s_pick) {
  const int tid = threadIdx.x;
  if (tid == 0) *s_pick = 0x7fffffff;
  double own[kQuarters], bef[kQuarters];
#pragma unroll
  for (int q = 0; q < kQuarters; ++q) own[q] = ((mass(4 * q) + mass(4 * q + 1)) + mass(4 * q + 2)) + mass(4 * q + 3);
  block_excl_scan_runs(own, bef, s_w);
  int pick = 0x7fffffff;
#pragma unroll
  for (int q = 0; q < kQuarters; ++q) {
    const double bf = pre + bef[q];
    if (pick == 0x7fffffff && bf + own[q] > target && !(bf > target)) {
      double run = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        run += mass(4 * q + j);
        if (pick == 0x7fffffff && bf + run > target) pick = slot_tok(c0, 4 * q + j);
      }
    }
  }
  if (pick != 0x7fffffff) atomicMin(s_pick, pick);  // rounding may let two runs both claim it
  __syncthreads();
  int k = *s_pick;
  __syncthreads();
  if (k != 0x7fffffff) return k;
  int best = -1;
#pragma unroll
  for (int s2 = 0; s2 < kPer; ++s2)
    if (mass(s2) > 0.0) best = max(best, slot_tok(c0, s2));
  best = wave_max_i(best);
  if (tid == 0) *s_pick = -1;
  __syncthreads();
  if ((tid & 63) == 0) atomicMax(s_pick, best);
  __syncthreads();
  k = *s_pick;
  __syncthreads();
  return k;
}

// LDS of a request's walk.
struct WalkLds {
  NodeRes res[64];
  int oacc[64], oterm[64], tok[64], pn[64], ot[64], len;
};
// The request's last reported node walks from the root: it reads every node's
// result, writes accepted_child / term_token and, when asked, the accepted path
// (what spec_accept_path derives from them, produced by the same walk), and leaves
// the request counter and the nodes' error words at zero for the next call.
// verdict: the request's tree verdict.  Called by the whole workgroup.
__device__ void request_walk(const RejArgs& a, const SampWs& w, int b, int verdict, int nb, WalkLds* L) {
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)b * a.n_max;
  if (tid < 64) {
    const bool in = tid < a.n_max;
    L->res[tid].acc = in ? pub_load(&w.res[base + tid].acc) : SPEC_NODE_NOT_EVALUATED;
    L->res[tid].term = in ? pub_load(&w.res[base + tid].term) : SPEC_NODE_NOT_EVALUATED;
    L->res[tid].err = in ? pub_load(&w.res[base + tid].err) : 0;
    L->tok[tid] = in ? a.tokens[base + tid] : 0;
    L->oacc[tid] = L->oterm[tid] = SPEC_NODE_NOT_EVALUATED;
    L->pn[tid] = L->ot[tid] = -1;
  }
  __syncthreads();
  if (tid < a.n_max && L->res[tid].err) pub_store(&w.res[base + tid].err, 0);
  if (tid == 0) {
    pub_store(&w.req_count[b], 0u);
    int vd = verdict, cur = 0, len = 0;
    bool bad = false;
    L->pn[0] = 0;
    for (int step = 0; vd == 0 && step < nb; ++step) {
      const NodeRes r = L->res[cur];
      if (r.err) {
        vd = (r.err & 2) ? SPEC_ERR_TIMEOUT : SPEC_ERR_BAD_INPUT;
        break;
      }
      L->oacc[cur] = r.acc;
      if (r.acc >= 0) {  // a child of cur: index above cur, below nb
        cur = r.acc;
        ++len;
        L->pn[len] = cur;
        L->ot[len - 1] = L->tok[cur];
        continue;
      }
      L->oterm[cur] = r.term;
      if (r.term < 0) {
        report(a.status, SPEC_ERR_BAD_INPUT);
        bad = true;
      } else {
        L->ot[len] = r.term;
      }
      break;
    }
    if (vd != 0) {
      for (int i = 0; i < 64; ++i) L->oacc[i] = L->oterm[i] = SPEC_NODE_NOT_EVALUATED;
      L->oacc[0] = SPEC_NODE_BAD_REQUEST;
      report(a.status, vd);
    }
    if (vd != 0 || bad) {  // no path
      for (int i = 0; i < 64; ++i) L->pn[i] = L->ot[i] = -1;
      len = -1;
    }
    L->len = len;
  }
  __syncthreads();
  if (tid < a.n_max) {
    a.accepted_child[base + tid] = L->oacc[tid];
    a.term_token[base + tid] = L->oterm[tid];
    if (a.path_nodes) {
      a.path_nodes[base + tid] = L->pn[tid];
      a.out_tokens[base + tid] = L->ot[tid];
    }
  }
  if (tid == 0 && a.path_nodes) a.accept_len[b] = L->len;
}


// One wavefront merges a row's chunk partials in chunk order: m = max_c m_c,
// Z = sum_c s_c exp((m_c - m) / T); a NaN chunk maximum (a chunk holding NaN or
// +inf) or an all -inf row makes the row invalid.
__device__ inline void merge_row(const float* cm, const double* cs, int nch, double inv, float* m_out, double* z_out,
                                 int* ok_out) {
  const int lane = threadIdx.x & 63;
  constexpr int kC = 4;  // chunks per lane (256 at most)
  float mc[kC];
  double sc[kC];
#pragma unroll
  for (int j = 0; j < kC; ++j) {
    const int c = lane + 64 * j;
    mc[j] = c < nch ? cm[c] : -INFINITY;
    sc[j] = c < nch ? cs[c] : 0.0;
  }
  int bad = 0;
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kC; ++j) {
    bad |= isnan(mc[j]) ? 1 : 0;
    mx = fmaxf(mx, mc[j]);
  }
  bad = wave_or_i(bad);
  const float m = wave_max_f(mx);
  double z = 0.0;
#pragma unroll
  for (int j = 0; j < kC; ++j) {
    const int c = lane + 64 * j;
    if (!bad && c < nch && mc[j] > -INFINITY) z += sc[j] * exp(((double)mc[j] - (double)m) * inv);
  }
  z = wave_sum_d(z);
  *m_out = m;
  *z_out = z;
  *ok_out = !bad && m > -INFINITY && z > 0.0;
}


// Chunk holding the target u * sum(s_chunk[0 .. nch)) (nch <= blockDim.x); *pre is
// the mass of the chunks before it.
__device__ inline int pick_chunk(const double* s_chunk, int nch, double u, double* s_w, int* s_pick, double* pre,
                                 double* target) {
  const int tid = threadIdx.x;
  const double v = tid < nch ? s_chunk[tid] : 0.0;
  if (tid == 0) *s_pick = nch - 1;
  double S;
  const double before = block_excl_scan_d(v, s_w, &S);
  const double tg = u * S;
  if (tid < nch - 1 && before + v > tg) atomicMin(s_pick, tid);
  __syncthreads();
  const int ch = *s_pick;
  __syncthreads();
  *target = tg;
  // the prefix of the chosen chunk, as its owner computed it
  if (tid == ch) s_w[4] = before;
  __syncthreads();
  *pre = s_w[4];
  __syncthreads();
  return ch;
}


// T == 0: one wavefront per request follows the target argmax.
__global__ __launch_bounds__(64) void greedy_walk_kernel(GreedyArgs g) { greedy_walk_wave<false>(g, blockIdx.x); }


// ---------------------------------------------------------------------------
// The sampler: one workgroup per (node slot, vocabulary chunk)
// ---------------------------------------------------------------------------
// The chain's level step.  level_push (every wavefront, no barrier): the wavefront
// sums, exactly, the fixed-point masses of its tokens with dp - K dq > 0 (a thread's
// below 2^46, the wavefront's below 2^52: exact in fp64), adds them into the
// workgroup's accumulators of the level's parity (LDS atomics on exact integers, so
// the order of arrival does not matter) and takes a ticket; the last wavefront to
// arrive reads the chunk's sums (below 2^55), resets the accumulators and, with
// more than one chunk, publishes them as two words (sum << kTagBits) | level,
// through this XCD's L2 when the node's chunks share it (local), else device-wide.
// gather_level (wave 0): every chunk's words of the level, this chunk's included
// (lane l reads chunks l, l + 64, ...; each wait bounded by wait_limit polls) into
// s_lp / s_lq, their totals into s_tot; false when a wait gave up.
__device__ inline void level_push(const double* dp, const double* dq, double K, unsigned long long* sl0, int nch,
                                  int ch, int lv, int local, unsigned long long* s_acc, uint32_t* s_cnt,
                                  long long* s_own) {
  double sp = 0.0, sq = 0.0;
#pragma unroll
  for (int s2 = 0; s2 < kPer; ++s2) {
    const double in = __fma_rn(-K, dq[s2], dp[s2]) > 0.0 ? 1.0 : 0.0;
    sp = __fma_rn(in, dp[s2], sp);  // exact: integers below 2^53
    sq = __fma_rn(in, dq[s2], sq);
  }
  sp = wave_sum_d(sp);
  sq = wave_sum_d(sq);
  if ((threadIdx.x & 63) == 0) {
    const int par = lv & 1;
    __hip_atomic_fetch_add(&s_acc[2 * par], (unsigned long long)(long long)sp, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_add(&s_acc[2 * par + 1], (unsigned long long)(long long)sq, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint32_t t = __hip_atomic_fetch_add(&s_cnt[par], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (t == kThreads / 64 - 1) {
      const unsigned long long P = __hip_atomic_load(&s_acc[2 * par], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      const unsigned long long Q =
          __hip_atomic_load(&s_acc[2 * par + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_store(&s_acc[2 * par], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_store(&s_acc[2 * par + 1], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_store(&s_cnt[par], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (nch > 1) {
        unsigned long long* sl = sl0 + par * nch * 2;
        const unsigned long long wp = (P << kTagBits) | (unsigned)lv;
        const unsigned long long wq = (Q << kTagBits) | (unsigned)lv;
        if (local) {
          __hip_atomic_store(&sl[2 * ch], wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          __hip_atomic_store(&sl[2 * ch + 1], wq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        } else {
          pub_store(&sl[2 * ch], wp);
          pub_store(&sl[2 * ch + 1], wq);
        }
      } else {  // one chunk: its sums are the node's, handed to the gather through LDS
        __hip_atomic_store(&s_own[2 * par], (long long)P, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_store(&s_own[2 * par + 1], (long long)Q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_store(&s_cnt[2 + par], (uint32_t)lv, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
}
__device__ inline bool gather_level(const unsigned long long* sl0, int nch, int lv, uint32_t wait_limit, long long* s_lp,
                                    long long* s_lq, long long* s_tot, const uint32_t* s_cnt, const long long* s_own) {
  const int lane = threadIdx.x & 63;
  const unsigned long long* sl = sl0 + (lv & 1) * nch * 2;
  const unsigned tag = (unsigned)lv;
  long long cp = 0, cq = 0;
  bool ready = true;
  if (nch == 1) {  // the chunk's own sums, once its last wavefront has left them in LDS
    uint32_t polls = 0;
    while (__hip_atomic_load(&s_cnt[2 + (lv & 1)], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != (uint32_t)lv &&
           polls < wait_limit) {
      __builtin_amdgcn_s_sleep(1);
      ++polls;
    }
    ready = polls < wait_limit;
    if (lane == 0) {
      s_lp[0] = s_own[2 * (lv & 1)];
      s_lq[0] = s_own[2 * (lv & 1) + 1];
      s_tot[0] = s_own[2 * (lv & 1)];
      s_tot[1] = s_own[2 * (lv & 1) + 1];
    }
    return __ballot(!ready) == 0;
  }
  for (int t = lane; t < nch; t += 64) {
    unsigned long long xp = pub_load(&sl[2 * t]), xq = pub_load(&sl[2 * t + 1]);
    for (uint32_t polls = 0; ((xp & 0xffu) != tag || (xq & 0xffu) != tag) && polls < wait_limit; ++polls) {
      __builtin_amdgcn_s_sleep(1);
      xp = pub_load(&sl[2 * t]);
      xq = pub_load(&sl[2 * t + 1]);
    }
    ready = ready && (xp & 0xffu) == tag && (xq & 0xffu) == tag;
    const long long vp = (long long)(xp >> kTagBits), vq = (long long)(xq >> kTagBits);
    s_lp[t] = vp;
    s_lq[t] = vq;
    cp += vp;
    cq += vq;
  }
  cp = wave_sum_ll(cp);
  cq = wave_sum_ll(cq);
  if (lane == 0) {
    s_tot[0] = cp;
    s_tot[1] = cq;
  }
  return __ballot(!ready) == 0;
}

// Workgroup blockIdx = nx i + x serves group x (with nx = the XCD count, the hardware
// dispatches it to one XCD): the nodes of ordinal o = nx g + x, in blocks of nb_blk
// nodes.  Ordinals run over node slots first and requests second (o = n batch + b),
// so every request's first slots (the root and the nodes nearest it, which hold the
// long sibling chains; the later slots are mostly leaves) start ahead of the later
// slots.  A block's workgroups are first one planner per node (ch = -1: the plan, a
// leaf's draw, the report of a node that needs no chain; it never waits), then the
// nch chunks of each node, node by node.  Only the chunks of one node wait, and only
// for each other; workgroups start in blockIdx order, so the first unfinished node
// always has all of its chunks started, and every wait ends.  *nd = batch n_max for an
// ordinal past the last node.
__device__ inline void chunk_of(int blk, int q_off, int nch, int nx, int nb_blk, int batch, int n_max, int* nd,
                                int* ch) {
  const int x = blk % nx, q = blk / nx + q_off;
  const int per = nb_blk * (nch + 1), blkno = q / per, r = q % per;
  int g, c;
  if (r < nb_blk) {
    g = blkno * nb_blk + r;
    c = -1;
  } else {
    const int h = r - nb_blk;
    g = blkno * nb_blk + h / nch;
    c = h % nch;
  }
  const int o = g * nx + x;
  *nd = o < batch * n_max ? (o % batch) * n_max + o / batch : batch * n_max;
  *ch = c;
}

// Six waves per SIMD: three workgroups per CU (80 VGPRs; a few registers spill to
// scratch), so more of a batch's chunks are resident at once.
__global__ __launch_bounds__(kThreads, 6) void sample_kernel(RejArgs a, SampWs w, uint32_t wait_limit, int nx,
                                                             int nb_blk, int q_off, int local) {
  __shared__ int s_par[64], s_tok[64];
  __shared__ float s_ua[64];
  __shared__ double s_px[64], s_qx[64];
  __shared__ float s_cm[256];
  __shared__ double s_pch[256], s_chunk[256];
  __shared__ long long s_lp[2][256], s_lq[2][256];  // every chunk's sums at the last two levels
  __shared__ double s_w[16];
  __shared__ long long s_tot[2], s_own[4];
  __shared__ unsigned long long s_acc[4];  // a level's chunk sums, by level parity
  __shared__ uint32_t s_cnt[4];            // arrivals by parity; [2 + parity]: the level whose own sums are in s_own
  __shared__ double s_z[2];
  __shared__ float s_m[2];
  __shared__ int s_ok[2], s_nb, s_pick, s_fail, s_done, s_last;
  __shared__ WalkLds s_walk;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nch = a.nch, nodes = a.batch * a.n_max;
  int nd, ch;
  chunk_of((int)blockIdx.x, q_off, nch, nx, nb_blk, a.batch, a.n_max, &nd, &ch);
  if (nd >= nodes) return;
  const bool planner = ch < 0;
  const int b = nd / a.n_max, n = nd % a.n_max;
  const int64_t base = (int64_t)b * a.n_max, row = nd;
  // ---- round 1.  Every wavefront reads the request's parent links (lane = node
  // slot): a node without children has nothing for its other chunks, and an
  // internal node's chunk of both rows is in flight from here on (kept in
  // registers).  Wave 0 also reads the tokens and uniforms, checks the tree and
  // fetches the children's tested logits; waves 1 and 2 merge the node's target
  // and draft row statistics from the chunk partials; wave 3 keeps the target chunk
  // partials for a draw from p ----
  const bool in = lane < a.n_max;
  const int par = in ? a.parent[base + lane] : -2;
  const int nb = a.n_nodes[b];
  const bool n_ok = nb >= 1 && nb <= a.n_max;
  const bool live = n_ok && lane < nb;
  const bool has_kids = n_ok && n < nb && __ballot(live && lane > 0 && par == n) != 0;
  if (!planner && !has_kids) return;
  float xl[kPer], xd[kPer];
  if (!planner && has_kids) {
    load_chunk(a.tgt_logits + row * a.vocab, ch * kChunk, a.vocab, a.vec, xl);
    load_chunk(a.dft_logits + row * a.vocab, ch * kChunk, a.vocab, a.vec, xd);
  }
  float lt_kid = 0.0f, ld_kid = 0.0f;  // wave 0: the tested token's logits of the child in this lane
  if (wv == 0) {
    const int tk = in ? a.tokens[base + lane] : 0;
    s_par[lane] = par;
    s_tok[lane] = tk;
    s_ua[lane] = in ? a.u_accept[base + lane] : 0.0f;
    if (lane == 0) s_fail = 0;
    if (lane < 4) {
      s_acc[lane] = 0ull;
      s_cnt[lane] = 0u;
    }
    const bool bad_link = live && (lane == 0 ? par != -1 : (par < 0 || par >= lane));
    const bool bad_tok = live && lane > 0 && (tk < 0 || tk >= a.vocab);
    if (!__ballot(bad_link) && !__ballot(bad_tok) && live && lane > 0 && par == n) {
      lt_kid = a.tgt_logits[row * a.vocab + tk];
      ld_kid = a.dft_logits[row * a.vocab + tk];
    }
  } else if (wv <= 2) {
    const bool tg = wv == 1;
    float m;
    double z;
    int ok;
    merge_row((tg ? a.tgt_chunk_max : a.dft_chunk_max) + row * nch, (tg ? a.tgt_chunk_sum : a.dft_chunk_sum) + row * nch,
              nch, tg ? a.inv_t : a.inv_td, &m, &z, &ok);
    if (lane == 0) {
      s_m[wv - 1] = m;
      s_z[wv - 1] = z;
      s_ok[wv - 1] = ok;
    }
  } else if (wv == 3) {
    for (int c = lane; c < nch; c += 64) {
      s_cm[c] = a.tgt_chunk_max[row * nch + c];
      s_pch[c] = a.tgt_chunk_sum[row * nch + c];
    }
  }
  const float us = a.u_sample[row];
  __syncthreads();
  // ---- tree verdict and this node's children, in every wavefront ----
  const int tok = s_tok[lane];
  const bool bad_link = live && (lane == 0 ? par != -1 : (par < 0 || par >= lane));
  const bool bad_tok = live && lane > 0 && (tok < 0 || tok >= a.vocab);
  const unsigned long long m_link = __ballot(bad_link), m_tok = __ballot(bad_tok);
  const int verdict = (!n_ok || m_link) ? SPEC_ERR_BAD_TREE : (m_tok ? SPEC_ERR_BAD_INPUT : 0);
  const bool is_kid = verdict == 0 && live && lane > 0 && par == n;
  const uint64_t kids = __ballot(is_kid);
  const int k = __popcll(kids);
  const bool node_ok = verdict == 0 && n < nb;
  // a leaf needs only its target row: its draft row takes no part (parts C and G)
  const bool row_ok = s_ok[0] && (k == 0 || s_ok[1]);
  const float mt = s_m[0], md = s_m[1];
  const double izt = row_ok ? 1.0 / s_z[0] : 0.0, izd = row_ok ? 1.0 / s_z[1] : 0.0;
  const bool internal = node_ok && row_ok && k > 0;
  if (!planner && !internal) return;  // only an internal node needs its chunks
  // ---- a chunk of an internal node: its fixed-point masses as exact fp64 integers
  // (below 2^43).  A token belongs to W(c) when dp - K dq > 0 with K = c Z_t / Z_d
  // (the same expression in every chunk and in the terminal scan).  The level-1 sums
  // (threshold 1, whatever the first child's test gives) start at once ----
  double dp[kPer], dq[kPer];
  const double kr = izd / izt;  // K = c kr
  unsigned long long* sl0 = w.slot + (int64_t)nd * 4 * nch;
  if (!planner) {
#pragma unroll
    for (int s2 = 0; s2 < kPer; ++s2) {
      dp[s2] = (double)fx42(exp_scaled(xl[s2] - mt, a.est));
      dq[s2] = (double)fx42(exp_scaled(xd[s2] - md, a.esd));
    }
    level_push(dp, dq, kr, sl0, nch, ch, 1, local, s_acc, s_cnt, s_own);
  }
  // the chunk masses of p
  if (row_ok)
    for (int c = tid; c < nch; c += kThreads) s_pch[c] *= exp(((double)s_cm[c] - (double)mt) * a.inv_t);
  __syncthreads();
  if (wv == 0) {
    // ---- round 2: the children's p and q (fp64) ----
    double px = 0.0, qx = 0.0;
    if (is_kid && row_ok) {
      px = exp(((double)lt_kid - (double)mt) * a.inv_t) * izt;
      qx = exp(((double)ld_kid - (double)md) * a.inv_td) * izd;
    }
    s_px[lane] = px;
    s_qx[lane] = qx;
  }
  __syncthreads();
  NodeRes res{SPEC_NODE_NOT_EVALUATED, SPEC_NODE_NOT_EVALUATED, 0, 0};
  int owner = -1;       // the workgroup that writes this node's result: the planner, or a chunk
  bool chain = false;   // the sibling chain runs (first child rejected)
  int lv = 0;           // levels summed
  bool failed = false;  // a wait gave up
  if (node_ok) {
    if (!row_ok) {
      res.err = 1;
    } else if (k == 0) {
      // ---- leaf: the bonus from p, in the chunk that holds the target ----
      double pre, target;
      const int cs = pick_chunk(s_pch, nch, (double)us, s_w, &s_pick, &pre, &target);
      load_chunk(a.tgt_logits + row * a.vocab, cs * kChunk, a.vocab, a.vec, xl);
      const float mc = s_cm[cs];
      const double scale = exp(((double)mc - (double)mt) * a.inv_t);
      res.acc = SPEC_NODE_NONE;
      res.term = regs_scan([&](int s2) { return (double)exp_scaled(xl[s2] - mc, a.est) * scale; }, cs * kChunk, pre,
                           target, s_w, &s_pick);
    } else {
      const int fc = __ffsll((unsigned long long)kids) - 1;
      if (sibling_accepts(s_ua[fc], s_px[fc], s_qx[fc], 0.0, 1.0)) {
        res.acc = fc;  // the planner reports it; the chunks only clear their words
      } else if (planner) {
        return;  // the node's chunks follow its sibling chain and report it
      } else {
        // ---- the sibling chain: children after the first, in ascending index ----
        chain = true;
        owner = 0;
        double c = 0.0, W = 1.0;
        bool zero = false;  // the last step found no mass: the residual keeps its threshold
        int acc = SPEC_NODE_NONE, good = -1;  // good: parity of the level whose sums define c
        uint64_t rest = kids & (kids - 1);
        lv = 1;  // level 1's sums are out already
        while (true) {
          if (!zero) {
            // the child just tested was rejected: the threshold after it is c + W
            const double cn = c + W;
            if (lv > 1) level_push(dp, dq, cn * kr, sl0, nch, ch, lv, local, s_acc, s_cnt, s_own);
            if (wv == 0 && !gather_level(sl0, nch, lv, wait_limit, s_lp[lv & 1], s_lq[lv & 1], s_tot, s_cnt, s_own))
              s_fail = 1;
            __syncthreads();
            if (s_fail) {
              failed = true;
              break;
            }
            const double Wn = ((double)s_tot[0] * izt - cn * (double)s_tot[1] * izd) * kFxInv;
            if (Wn > 0.0) {
              c = cn;
              W = Wn;
              good = lv & 1;
            } else {
              zero = true;
            }
          }
          if (!rest) break;  // every child rejected
          const int ci = __ffsll((unsigned long long)rest) - 1;
          rest &= rest - 1;
          if (sibling_accepts(s_ua[ci], s_px[ci], s_qx[ci], c, W)) {
            acc = ci;
            break;
          }
          if (!zero) ++lv;
        }
        res.acc = acc;
        if (acc < 0 && !failed) {
          // ---- every child rejected: the bonus from the residual max(0, p - c q) ----
          double pre, target;
          if (good < 0) {  // no step changed the residual: it is p
            owner = pick_chunk(s_pch, nch, (double)us, s_w, &s_pick, &pre, &target);
            if (ch == owner) {
              const float mc = s_cm[ch];
              const double scale = exp(((double)mc - (double)mt) * a.inv_t);
              res.term = regs_scan([&](int s2) { return (double)exp_scaled(xl[s2] - mc, a.est) * scale; }, ch * kChunk,
                                   pre, target, s_w, &s_pick);
            }
          } else {
            for (int t = tid; t < nch; t += kThreads)
              s_chunk[t] = ((double)s_lp[good][t] * izt - c * (double)s_lq[good][t] * izd) * kFxInv;
            __syncthreads();
            owner = pick_chunk(s_chunk, nch, (double)us, s_w, &s_pick, &pre, &target);
            if (ch == owner) {
              const double K = c * kr, sc = izt * kFxInv;
              res.term = regs_scan([&](int s2) { return fmax(0.0, __fma_rn(-K, dq[s2], dp[s2])) * sc; }, ch * kChunk,
                                   pre, target, s_w, &s_pick);
            }
          }
        }
      }
    }
  }
  if (tid == 0) {
    if (failed) {
      report(a.status, SPEC_ERR_TIMEOUT);
      atomicAdd(&w.diag[kDiagTimeouts], 1u);
      atomicOr(&w.res[nd].err, 2);
    }
    if (ch == 0 && lv > 0) atomicAdd(&w.diag[kDiagLevels], (uint32_t)lv);
    if (ch == owner) {
      pub_store(&w.res[nd].acc, res.acc);
      pub_store(&w.res[nd].term, res.acc >= 0 ? SPEC_NODE_NOT_EVALUATED : res.term);
      if (res.err) atomicOr(&w.res[nd].err, res.err);
    }
  }
  // ---- the chunks of an internal node published level words: the last of them to
  // finish clears them (after reporting a chain node).  A chain node is reported by
  // that chunk, any other node by its planner ----
  const bool words = !planner && nch > 1;
  if (words) {
    if (tid == 0) {
      stores_done();
      s_done = pub_arrive(&w.exit_count[nd]) == (uint32_t)(nch - 1);
    }
    __syncthreads();
    if (!s_done) return;
    if (tid == 0) pub_store(&w.exit_count[nd], 0u);
  }
  if (planner || chain) {
    if (tid == 0) {
      stores_done();
      s_last = pub_arrive(&w.req_count[b]) == (uint32_t)(a.n_max - 1);
    }
    __syncthreads();
  }
  if (words)
    for (int t = tid; t < 4 * nch; t += kThreads) pub_store(&sl0[t], 0ull);
  if ((planner || chain) && s_last) request_walk(a, w, b, verdict, nb, &s_walk);
}

}  // namespace spectree

// ---- host side ----
namespace spectree {

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout: counters, node results, plans and the tagged level words.
inline size_t samp_ws_layout(int64_t batch, int64_t nodes, int nch, char* base, SampWs* w) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += a256(bytes);
    return p;
  };
  SampWs t{};
  t.diag = (uint32_t*)take(16);
  t.res = (NodeRes*)take((size_t)nodes * sizeof(NodeRes));
  t.req_count = (uint32_t*)take((size_t)batch * 4);
  t.exit_count = (uint32_t*)take((size_t)nodes * 4);
  t.slot = (unsigned long long*)take((size_t)nodes * 4 * nch * 8);
  if (w) *w = t;
  return off;
}

uint32_t g_wait_limit = kWaitDefault;

// The current device's XCD count and how many sampler workgroups all its CUs hold at
// once (from the runtime's occupancy query; both cached per device).
struct DevShape {
  int xcds, resident;
};
inline DevShape dev_shape() {
  static DevShape cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DevShape{1, 0};
  if (!cached[dev].resident) {
    int n = 0, cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n < 1) n = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sample_kernel, kThreads, 0) != hipSuccess) per_cu = 0;
    cached[dev] = DevShape{n, std::max(1, cus * per_cu)};
  }
  return cached[dev];
}

}  // namespace spectree

extern "C" size_t spec_tree_reject_sample_workspace_size(int32_t batch, int32_t n_max, int32_t vocab) {
  using namespace spectree;
  if (batch < 1 || n_max < 1 || n_max > 64 || vocab < 1) return 0;
  const int nch = (vocab + kChunk - 1) / kChunk;
  return samp_ws_layout(batch, (int64_t)batch * n_max, nch, nullptr, nullptr);
}

extern "C" void spec_tree_reject_sample_set_wait_limit(uint32_t polls) {
  spectree::g_wait_limit = polls ? polls : spectree::kWaitDefault;
}

extern "C" int spec_tree_reject_sample(const float* tgt_logits, float temperature, const float* tgt_max,
                                       const int32_t* tgt_argmax, const float* tgt_chunk_max,
                                       const double* tgt_chunk_sum, const float* dft_logits,
                                       float draft_temperature, const float* dft_chunk_max,
                                       const double* dft_chunk_sum, const int32_t* tokens, const int32_t* parent,
                                       const int32_t* n_nodes, const float* u_accept, const float* u_sample,
                                       int32_t batch, int32_t n_max, int32_t vocab, int32_t* accepted_child,
                                       int32_t* term_token, int32_t* path_nodes, int32_t* out_tokens,
                                       int32_t* accept_len, void* workspace, size_t workspace_bytes,
                                       int32_t* status, void* stream) {
  using namespace spectree;
  if (!(temperature >= 0.0f) || isinf(temperature)) return SPEC_ERR_INVALID_ARG;
  const bool greedy = temperature == 0.0f;
  if (!tgt_logits || !tokens || !parent || !n_nodes || !accepted_child || !term_token) return SPEC_ERR_INVALID_ARG;
  if ((path_nodes == nullptr) != (out_tokens == nullptr) || (path_nodes == nullptr) != (accept_len == nullptr))
    return SPEC_ERR_INVALID_ARG;  // the path outputs come together
  if (greedy && (!tgt_max || !tgt_argmax)) return SPEC_ERR_INVALID_ARG;
  if (!greedy) {
    if (!tgt_chunk_max || !tgt_chunk_sum || !dft_logits || !dft_chunk_max || !dft_chunk_sum || !u_accept ||
        !u_sample)
      return SPEC_ERR_INVALID_ARG;
    if (!(draft_temperature > 0.0f) || isinf(draft_temperature)) return SPEC_ERR_INVALID_ARG;
  }
  if (batch < 1 || n_max < 1 || n_max > 64 || vocab < 1) return SPEC_ERR_INVALID_ARG;
  const int nch = (vocab + kChunk - 1) / kChunk;
  if (nch > 256) return SPEC_ERR_UNSUPPORTED;
  RejArgs a{};
  a.tgt_logits = tgt_logits;
  a.dft_logits = dft_logits;
  a.tgt_max = tgt_max;
  a.tgt_argmax = tgt_argmax;
  a.tgt_chunk_max = tgt_chunk_max;
  a.tgt_chunk_sum = tgt_chunk_sum;
  a.dft_chunk_max = dft_chunk_max;
  a.dft_chunk_sum = dft_chunk_sum;
  a.inv_t = greedy ? 0.0 : 1.0 / (double)temperature;
  a.inv_td = greedy ? 0.0 : 1.0 / (double)draft_temperature;
  a.est = make_exp_scale(a.inv_t);
  a.esd = make_exp_scale(a.inv_td);
  a.tokens = tokens;
  a.parent = parent;
  a.n_nodes = n_nodes;
  a.u_accept = u_accept;
  a.u_sample = u_sample;
  a.batch = batch;
  a.n_max = n_max;
  a.vocab = vocab;
  a.nch = nch;
  a.vec = (vocab % 4 == 0) && (((uintptr_t)tgt_logits & 15) == 0) && (greedy || (((uintptr_t)dft_logits & 15) == 0));
  a.accepted_child = accepted_child;
  a.term_token = term_token;
  a.path_nodes = path_nodes;
  a.out_tokens = out_tokens;
  a.accept_len = accept_len;
  a.status = status;
  hipStream_t st = (hipStream_t)stream;
  if (greedy) {
    const GreedyArgs g{parent, tokens, n_nodes, tgt_max, tgt_argmax, n_max, vocab, accepted_child, term_token,
                       path_nodes, out_tokens, accept_len, status};
    hipLaunchKernelGGL(greedy_walk_kernel, dim3((unsigned)batch), dim3(64), 0, st, g);
    SPEC_LAUNCH_CHECK();
    return SPEC_OK;
  }
  const int64_t nodes = (int64_t)batch * n_max;
  if (!workspace || workspace_bytes < samp_ws_layout(batch, nodes, nch, nullptr, nullptr)) return SPEC_ERR_WORKSPACE;
  SampWs w{};
  samp_ws_layout(batch, nodes, nch, (char*)workspace, &w);
  // a node's chunks on one XCD when they fit there beside a block's plans, else over
  // the whole device; blocks of nb_blk nodes per group (see chunk_of)
  const DevShape ds = dev_shape();
  int nx = ds.xcds, cap = ds.resident / nx;
  if (nch > kLocalMaxChunks || cap < nch + 8) {
    nx = 1;
    cap = ds.resident;
  }
  if (cap < nch) return SPEC_ERR_UNSUPPORTED;  // one node's chunks must run together
  const int local = nx > 1 ? 1 : 0;
  const int64_t per_group = (nodes + nx - 1) / nx;
  const int nb_blk = (int)std::min<int64_t>(std::max(1, cap / 2), per_group);
  // whole blocks per launch, the work-items of one launch below 2^31
  const int64_t per = (int64_t)nb_blk * (nch + 1), rows = (per_group + nb_blk - 1) / nb_blk * per;
  const int64_t max_rows = std::max<int64_t>(1, ((int64_t)1 << 31) / ((int64_t)kThreads * nx * per)) * per;
  if (rows > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  for (int64_t q0 = 0; q0 < rows; q0 += max_rows) {
    const int64_t n_rows = std::min(max_rows, rows - q0);
    hipLaunchKernelGGL(sample_kernel, dim3((unsigned)(nx * n_rows)), dim3(kThreads), 0, st, a, w, g_wait_limit, nx,
                       nb_blk, (int)q0, local);
    SPEC_LAUNCH_CHECK();
  }
  return SPEC_OK;
}
