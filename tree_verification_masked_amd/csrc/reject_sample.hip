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
// one token plus the scalars (c_j, W(c_j)).  Only tokens with ratio rho = p/q > c
// enter W(c), and c >= 1 after the first rejection.
//
// Every node is evaluated in parallel (the uniforms are indexed by node and child,
// so a node's outcome does not depend on how the walk reached it); the walk from
// the root then only follows the per-node results.  Launches (T > 0):
//   P   one workgroup per node: the row statistics of the node's target and draft
//       rows, merged from the logit pass's chunk partials (max and sum of
//       exponentials), its children and their tested tokens' p and q (fp64), its
//       first-child test, and the list of nodes whose first child is rejected
//       ("active": only they need W(c)).
//   R1  (two or more vocabulary chunks) every (active node, 4096-token chunk):
//       histogram of rho over 128 buckets per octave on [1, 16), two more just
//       below 1 and one for rho >= 16 or q == 0, with exact fixed-point sums of p
//       and q per bucket, merged per node with integer atomics.  The bucket comes
//       from an fp32 log-domain estimate whose error is far below the 1% of a
//       bucket assumed everywhere.
//   R2  the same items: from the merged histogram, rigorous intervals
//       I_l = [a_l, b_l] holding c_{l+1} for every level l (every workgroup of a
//       node derives the same ones); then exact sums of p and q over tokens with
//       rho above each interval, the few tokens inside an interval in a per-node
//       list, and per-chunk sums for the terminal draw.  Only tokens in buckets
//       that straddle an interval end get an exact fp64 ratio.
//   R3  one workgroup per node: sibling tests with exact W(c_j) from R2's sums and
//       list (the thresholds c_j follow from the rejections alone, so they are
//       computed first and the tests then run side by side), terminal draws
//       located by exact chunk sums and one chunk scan; the
//       last workgroup of a request walks from the root and writes the outputs.
//       Each node clears the chain state it consumed, so the next call finds the
//       workspace ready without any cross-workgroup wait.
// Masses are summed as exact integers: the fp32 unnormalised mass exp((l - m)/T)
// in [0, 1] is truncated to a multiple of 2^-42 (bit arithmetic, no rounding), so
// the sums are exact, independent of summation order and bitwise reproducible;
// the normalisation 1/Z is applied once to each sum.  Small vocabularies (one
// chunk) and any case outside the fast path's guarantees (list or queue overflow,
// threshold beyond the histogram range, zero-mass steps) take direct vocabulary
// passes in R3.
#include "common.hpp"

namespace spectree {

constexpr int kHB = 512;            // ratio buckets over [1, 16): 128 per octave
constexpr int kHLow = 2;            // buckets just below rho = 1
constexpr int kHTop = kHB + kHLow;  // rho >= 16 or q == 0
constexpr int kHN = kHTop + 1;
constexpr float kHMargin = 0.01f;   // bound on the estimate's error, in buckets
constexpr int kMaxKids = 63;        // chain levels per node
constexpr int kListCap = 4096;      // exact in-interval tokens kept per node
constexpr int kWgList = 256;        // in-interval tokens one R2 workgroup can stage
constexpr int kQueue = 1024;        // edge tokens one R2 workgroup can stage
constexpr int kLdsList = 512;       // list entries R3 keeps in LDS
constexpr int kShortList = 32;      // lists R3 walks with a single lane
constexpr int kMaxEdge = 24;        // edge buckets per level before the direct path
constexpr double kFx = 4398046511104.0;  // 2^42
constexpr double kFxInv = 1.0 / kFx;
constexpr int kRjThreads = 256;
constexpr int kFlagFallback = 1;

struct ListEntry {  // a token inside some interval
  long long fp, fq; // fixed-point unnormalised masses
  double rho;
  int32_t tok, pad;
};
struct QEntry {
  int32_t tok, h;
  float pp, qq;  // unnormalised fp32 masses
};
struct NodeRes {
  int32_t acc, term, err, pad;
};
struct NodeInfo {     // written by P for every node slot
  uint64_t kids;      // bit c: node c is a child
  int32_t active;     // first child rejected: the chain is needed
  int32_t verdict;    // the request's tree / token verdict (0 = fine)
  float K;            // log2(Z_d / Z_t), the bucket estimate's row constant
  float mt, md;       // row maxima of the target and draft rows (NaN: invalid row)
  int32_t pad;
  double izt, izd;    // 1 / Z_t, 1 / Z_d
};
struct KidInfo {      // tested token of a child: p(x), q(x) at its parent's row
  double px, qx;
};
struct ChainRec {     // R2 -> R3
  double a[kMaxKids], b[kMaxKids];
  int32_t flags, pad;
};
// Per-bucket table of R2: certain ratio range lb <= rho < ub of the bucket's tokens
// and the suffix sums of the merged histogram from this bucket up.
struct BucketRec {
  double lb, ub;
  long long SP, SQ;
};

constexpr int kDiagDirect = 0;  // diagnostics word: nodes finished by direct vocabulary passes

struct NodeWs {            // nd = b * n_max + n
  uint32_t* diag;          // [4]           cumulative counters (kDiag*)
  NodeRes* res;            // [nd]          R3 -> its request's last workgroup
  uint32_t* req_count;     // [batch]       self-resetting
  NodeInfo* info;          // [nd]          P -> R1, R2, R3
  KidInfo* kid;            // [nd]          P -> R3
  uint32_t* act_count;     // [1]           P -> R1, R2 (cleared by R3)
  int32_t* act_list;       // [nd]          P -> R1, R2
  long long* hist;         // [nd][kHN][2]  R1 -> R2 (cleared by R3)
  ChainRec* rec;           // [nd]          R2 -> R3 (flags cleared by R3)
  long long* lvl;          // [nd][kMaxKids][2]  R2 -> R3 (cleared by R3)
  long long* cdraw;        // [nd][nch][2]  R2 -> R3
  ListEntry* list;         // [nd][kListCap]     R2 -> R3
  uint32_t* list_n;        // [nd]          R2 -> R3 (cleared by R3)
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

// A thread's 16 tokens of a chunk held in registers.  Chunk layout (R1, R2): token
// of slot s is c0 + ((s / 4) * 256 + tid) * 4 + s % 4, so each 16-byte load of a
// wave covers 1 KB of consecutive tokens; all loads are issued before use.
constexpr int kPer = kChunk / 256;
__device__ inline int chunk_tok(int c0, int s) { return c0 + ((s >> 2) * 256 + (int)threadIdx.x) * 4 + (s & 3); }
__device__ inline void load_chunk(const float* row, int c0, int vocab, bool vec, float* x) {
  if (vec && c0 + kChunk <= vocab) {
#pragma unroll
    for (int k = 0; k < kPer / 4; ++k) {
      const float4 f = *reinterpret_cast<const float4*>(row + c0 + (k * 256 + (int)threadIdx.x) * 4);
      x[4 * k + 0] = f.x;
      x[4 * k + 1] = f.y;
      x[4 * k + 2] = f.z;
      x[4 * k + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int s2 = 0; s2 < kPer; ++s2) {
      const int t = chunk_tok(c0, s2);
      x[s2] = t < vocab ? row[t] : -INFINITY;
    }
  }
}
// R1 / R2 use 1024-thread workgroups: thread t holds tokens c0 + 4t .. c0 + 4t + 3.
constexpr int kCThreads = 1024;
constexpr int kCPer = kChunk / kCThreads;
__device__ inline void load_chunk4(const float* row, int c0, int vocab, bool vec, float* x) {
  const int t = c0 + 4 * (int)threadIdx.x;
  if (vec && t + 4 <= vocab) {
    const float4 f = *reinterpret_cast<const float4*>(row + t);
    x[0] = f.x;
    x[1] = f.y;
    x[2] = f.z;
    x[3] = f.w;
  } else {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) x[s2] = t + s2 < vocab ? row[t + s2] : -INFINITY;
  }
}
// R2 uses 512-thread workgroups (two per CU, so every item of a call is resident
// at once): thread t holds tokens c0 + 2048 j + 4t .. + 3 for j = 0, 1.
constexpr int kXThreads = 512;
constexpr int kXPer = kChunk / kXThreads;
static_assert(kXThreads == kHB && kXPer == 8, "R2 layout: one histogram bucket per thread below kHB");
__device__ inline int xtok(int c0, int s2) { return c0 + 2048 * (s2 >> 2) + 4 * (int)threadIdx.x + (s2 & 3); }
__device__ inline void load_chunk8(const float* row, int c0, int vocab, bool vec, float* x) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = c0 + 2048 * j + 4 * (int)threadIdx.x;
    if (vec && t + 4 <= vocab) {
      const float4 f = *reinterpret_cast<const float4*>(row + t);
      x[4 * j + 0] = f.x;
      x[4 * j + 1] = f.y;
      x[4 * j + 2] = f.z;
      x[4 * j + 3] = f.w;
    } else {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) x[4 * j + s2] = t + s2 < vocab ? row[t + s2] : -INFINITY;
    }
  }
}
// Contiguous layout (R3 scans): thread owns tokens r0 .. r0 + kPer - 1.
__device__ inline void load_run(const float* row, int r0, int t1, bool vec, float* x) {
  if (vec && r0 + kPer <= t1) {
#pragma unroll
    for (int k = 0; k < kPer / 4; ++k) {
      const float4 f = *reinterpret_cast<const float4*>(row + r0 + 4 * k);
      x[4 * k + 0] = f.x;
      x[4 * k + 1] = f.y;
      x[4 * k + 2] = f.z;
      x[4 * k + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int s2 = 0; s2 < kPer; ++s2) x[s2] = r0 + s2 < t1 ? row[r0 + s2] : -INFINITY;
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

struct RowView {
  const float* lt;
  const float* ld;
  float mt, md;
  double izt, izd;
};
// Exponent of the fp32 exp of the softmax kernel: exp_scaled(l - m) = 2^e.
__device__ inline float exp2_arg(float l, float m, ExpScale s) {
  const float d = fmaxf(l - m, -3.402823466e38f);
  return fmaf(d, s.hi, d * s.lo);
}
// Pass elements: the fp32 exp of the softmax kernel, normalised in fp64.
__device__ inline double p_el(const RejArgs& a, const RowView& r, float l) {
  return (double)exp_scaled(l - r.mt, a.est) * r.izt;
}
__device__ inline double q_el(const RejArgs& a, const RowView& r, float l) {
  return (double)exp_scaled(l - r.md, a.esd) * r.izd;
}
// Acceptance ratio r(x)/q(x) with r = max(0, p - c q) / W.
__device__ inline double accept_ratio(double px, double qx, double c, double W) {
  const double num = fmax(0.0, px - c * qx);
  if (qx > 0.0) return num / (W * qx);
  return num > 0.0 ? INFINITY : 0.0;
}

// ---------------------------------------------------------------------------
// Ratio buckets
// ---------------------------------------------------------------------------
// Bucket h of a token from the exponents of its two fp32 masses pp = 2^ep,
// qq = 2^eq and the row constant K = log2(Z_d / Z_t): h = floor(128 log2 rho~) + kHLow
// with log2 rho~ = ep - eq + K.  kHTop for rho~ >= 16 or qq == 0; -1 when pp == 0
// or rho~ < 2^(-2/128) (such tokens certainly have rho < 1).  The exact log2 rho
// differs from log2 rho~ by the exp2 and fp32 rounding, a few 1e-6 at most, far
// below kHMargin / 128: a token of bucket h has
//   2^((h - kHLow - kHMargin) / 128) <= rho < 2^((h - kHLow + 1 + kHMargin) / 128).
// R1 and R2 evaluate the same expression on the same inputs, with explicit
// rounding, so they always agree on h.
__device__ inline int est_bucket(float ep, float eq, float pp, float qq, float K) {
  float x = floorf(__fmul_rn(__fadd_rn(__fsub_rn(ep, eq), K), 128.0f));
  x = fminf(fmaxf(x, (float)(-kHLow - 1)), (float)kHB);  // NaN (both masses 0) becomes -3
  const int h = (int)x + kHLow;                           // -1 .. kHTop
  return pp > 0.0f ? (qq > 0.0f ? h : kHTop) : -1;
}
// Certain ratio range of each bucket: lb <= rho < ub (fp32 exp2 is within 2e-7
// relative, well inside the margin).  Entry kHN is a sentinel above every bucket.
__device__ inline void fill_edges(BucketRec* T) {
  for (int h = threadIdx.x; h <= kHN; h += blockDim.x) {
    const float beta = (float)(h - kHLow);
    if (h == kHN) {
      T[h].lb = INFINITY;
      T[h].ub = INFINITY;
    } else if (h == kHTop) {
      T[h].lb = (double)exp2f(((float)kHB - kHMargin) / 128.0f);
      T[h].ub = INFINITY;
    } else {
      T[h].lb = (double)exp2f((beta - kHMargin) / 128.0f);
      T[h].ub = (double)exp2f((beta + 1.0f + kHMargin) / 128.0f);
    }
  }
}
__device__ inline int bucket_guess(double c) {
  const int i = (int)floorf(log2f((float)c) * 128.0f) + kHLow;
  return min(max(i, 0), kHTop);
}
// First bucket all of whose tokens have rho > c (kHN if none).
__device__ inline int first_above(double c, const BucketRec* T) {
  int i = bucket_guess(c);
  while (i > 0 && T[i - 1].lb > c) --i;
  while (i < kHN && !(T[i].lb > c)) ++i;
  return i;
}
// First bucket that may hold a token with rho > c.
__device__ inline int first_maybe(double c, const BucketRec* T) {
  int i = bucket_guess(c);
  while (i > 0 && T[i - 1].ub > c) --i;
  while (i < kHN && !(T[i].ub > c)) ++i;
  return i;
}
// Bounds of W(c) from the merged histogram (fixed point of the unnormalised masses;
// p = P * izt * 2^-42): the buckets from ia = first_above(c) count in full, the one
// or two buckets [im, ia) straddling c contribute between max(0, P - cQ) (jointly)
// and (ub - c) Q each.  The six table entries around the fp32 guess of c's bucket
// are read at once; a guess that misses falls back to the scans above.
__device__ double w_bound(double c, const BucketRec* T, double izt, double izd, bool upper) {
  const int g = bucket_guess(c);
  const int base = min(max(g - 2, 0), kHN + 1 - 6);
  BucketRec r[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) r[j] = T[base + j];
  int ia = -1, im = -1;
#pragma unroll
  for (int j = 5; j >= 0; --j) {
    if (r[j].lb > c) ia = j;
    if (r[j].ub > c) im = j;
  }
  const bool ok = ia >= 0 && im >= 0 && (base == 0 || !(r[0].ub > c));
  if (!ok) {  // rare: scan the table
    const int A = first_above(c, T), M = first_maybe(c, T);
    const double full = ((double)T[A].SP * izt - c * (double)T[A].SQ * izd) * kFxInv;
    if (!upper) return full + fmax(0.0, ((double)(T[M].SP - T[A].SP) * izt - c * (double)(T[M].SQ - T[A].SQ) * izd) * kFxInv);
    double extra = 0.0;
    for (int h = M; h < A; ++h) {
      const double P = (double)(T[h].SP - T[h + 1].SP) * izt * kFxInv, Q = (double)(T[h].SQ - T[h + 1].SQ) * izd * kFxInv;
      extra += Q > 0.0 ? (isinf(T[h].ub) ? INFINITY : fmax(0.0, (T[h].ub - c) * Q)) : P;
    }
    return full + extra;
  }
  long long SPa = 0, SQa = 0, SPm = 0, SQm = 0;
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    if (j == ia) {
      SPa = r[j].SP;
      SQa = r[j].SQ;
    }
    if (j == im) {
      SPm = r[j].SP;
      SQm = r[j].SQ;
    }
  }
  const double full = ((double)SPa * izt - c * (double)SQa * izd) * kFxInv;
  if (!upper) return full + fmax(0.0, ((double)(SPm - SPa) * izt - c * (double)(SQm - SQa) * izd) * kFxInv);
  double extra = 0.0;
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    if (j >= im && j < ia) {
      const double P = (double)(r[j].SP - r[j + 1].SP) * izt * kFxInv;
      const double Q = (double)(r[j].SQ - r[j + 1].SQ) * izd * kFxInv;
      extra += Q > 0.0 ? (isinf(r[j].ub) ? INFINITY : fmax(0.0, (r[j].ub - c) * Q)) : P;
    }
  }
  return full + extra;
}

// The same bounds as w_bound, evaluated by a whole wavefront for a uniform c: lane j
// holds entry base + j of a 64-entry window around the guess, so the two bucket
// boundaries come from ballots and the sums from readlane; the terms are combined
// in the same order as in w_bound, so the result is identical.
__device__ double w_bound_wave(double c, const BucketRec* T, double izt, double izd, bool upper) {
  const int lane = threadIdx.x & 63;
  const int base = min(max(bucket_guess(c) - 16, 0), kHN + 1 - 64);
  const BucketRec r = T[base + lane];
  const uint64_t ma = __ballot(r.lb > c), mm = __ballot(r.ub > c);
  auto rl_ll = [](long long v, int l) {
    return (long long)(((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l));
  };
  auto rl_d = [&](double v, int l) { return __longlong_as_double(rl_ll(__double_as_longlong(v), l)); };
  if (!(ma && mm && (base == 0 || !(mm & 1ull)))) return w_bound(c, T, izt, izd, upper);  // rare
  const int ia = __ffsll((unsigned long long)ma) - 1, im = __ffsll((unsigned long long)mm) - 1;
  const long long SPa = rl_ll(r.SP, ia), SQa = rl_ll(r.SQ, ia);
  const double full = ((double)SPa * izt - c * (double)SQa * izd) * kFxInv;
  if (!upper) {
    const long long SPm = rl_ll(r.SP, im), SQm = rl_ll(r.SQ, im);
    return full + fmax(0.0, ((double)(SPm - SPa) * izt - c * (double)(SQm - SQa) * izd) * kFxInv);
  }
  double extra = 0.0;
  for (int h = im; h < ia; ++h) {
    const double P = (double)(rl_ll(r.SP, h) - rl_ll(r.SP, h + 1)) * izt * kFxInv;
    const double Q = (double)(rl_ll(r.SQ, h) - rl_ll(r.SQ, h + 1)) * izd * kFxInv;
    const double ub = rl_d(r.ub, h);
    extra += Q > 0.0 ? (isinf(ub) ? INFINITY : fmax(0.0, (ub - c) * Q)) : P;
  }
  return full + extra;
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

// ---------------------------------------------------------------------------
// P: per-node plan
// ---------------------------------------------------------------------------
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

// One workgroup (three waves) per node slot: wave 0 reads the request's tree and
// uniforms while waves 1 and 2 merge the node's target and draft rows; then wave 0
// finds the node's children, their tested tokens' p and q at this row (fp64, for
// R3) and the first-child test, and lists the node as active when that child is
// rejected (the list order is free: every node's outcome is its own).
__global__ __launch_bounds__(192) void plan_kernel(RejArgs a, NodeWs w, int chunked) {
  __shared__ int s_par[64], s_tok[64];
  __shared__ float s_ua[64];
  __shared__ double s_z[2];
  __shared__ float s_m[2];
  __shared__ int s_ok[2], s_nb;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nd = blockIdx.x;
  const int b = nd / a.n_max, n = nd % a.n_max;
  const int64_t base = (int64_t)b * a.n_max;
  if (wv == 0) {
    const bool in = lane < a.n_max;
    s_par[lane] = in ? a.parent[base + lane] : -2;
    s_tok[lane] = in ? a.tokens[base + lane] : 0;
    s_ua[lane] = in ? a.u_accept[base + lane] : 0.0f;
    if (lane == 0) s_nb = a.n_nodes[b];
  } else {
    const bool tg = wv == 1;
    float m;
    double z;
    int ok;
    merge_row((tg ? a.tgt_chunk_max : a.dft_chunk_max) + (int64_t)nd * a.nch,
              (tg ? a.tgt_chunk_sum : a.dft_chunk_sum) + (int64_t)nd * a.nch, a.nch, tg ? a.inv_t : a.inv_td, &m, &z,
              &ok);
    if (lane == 0) {
      s_m[wv - 1] = m;
      s_z[wv - 1] = z;
      s_ok[wv - 1] = ok;
    }
  }
  __syncthreads();
  if (wv != 0) return;
  const int nb = s_nb;
  const bool n_ok = nb >= 1 && nb <= a.n_max;
  const bool live = n_ok && lane < nb;
  const int par = s_par[lane], tok = s_tok[lane];
  const bool bad_link = live && (lane == 0 ? par != -1 : (par < 0 || par >= lane));
  const bool bad_tok = live && lane > 0 && (tok < 0 || tok >= a.vocab);
  const unsigned long long m_link = __ballot(bad_link), m_tok = __ballot(bad_tok);
  const int verdict = (!n_ok || m_link) ? SPEC_ERR_BAD_TREE : (m_tok ? SPEC_ERR_BAD_INPUT : 0);
  const bool tree_ok = verdict == 0;
  const bool row_ok = s_ok[0] && s_ok[1];
  const float mt = s_m[0], md = s_m[1];
  const double izt = row_ok ? 1.0 / s_z[0] : 0.0, izd = row_ok ? 1.0 / s_z[1] : 0.0;
  // the children of this node, and each one's tested token's p and q at this row
  const bool is_kid = tree_ok && live && lane > 0 && par == n;
  const uint64_t kids = __ballot(is_kid);
  double px = 0.0, qx = 0.0;
  if (is_kid && row_ok) {
    const int64_t o = (int64_t)nd * a.vocab + tok;
    px = exp(((double)a.tgt_logits[o] - (double)mt) * a.inv_t) * izt;
    qx = exp(((double)a.dft_logits[o] - (double)md) * a.inv_td) * izd;
  }
  if (is_kid) w.kid[base + lane] = KidInfo{px, qx};
  // first-child test of this node
  const int fc = kids ? __ffsll((unsigned long long)kids) - 1 : 0;
  const double fpx = __shfl(px, fc), fqx = __shfl(qx, fc);
  const bool active = tree_ok && n < nb && kids && row_ok && !((double)s_ua[fc] < accept_ratio(fpx, fqx, 0.0, 1.0));
  if (lane == 0) {
    NodeInfo inf;
    inf.kids = kids;
    inf.active = active;
    inf.verdict = verdict;
    inf.K = row_ok ? (float)(log2(s_z[1]) - log2(s_z[0])) : 0.0f;
    inf.mt = row_ok ? mt : NAN;
    inf.md = row_ok ? md : NAN;
    inf.pad = 0;
    inf.izt = izt;
    inf.izd = izd;
    w.info[nd] = inf;
    if (chunked && active) w.act_list[atomicAdd(w.act_count, 1u)] = nd;
  }
}

// ---------------------------------------------------------------------------
// R1: ratio histogram
// ---------------------------------------------------------------------------
// Items are (active node, group of cg consecutive chunks) pairs, item = slot *
// ngroups + group, visited grid-stride; a workgroup accumulates its group's chunks in
// LDS and merges them into the node's histogram with one set of integer atomics.
// Those atomics are what limits the launch when many nodes are active (every node's
// buckets receive one per group), so cg grows with the active (node, chunk) count --
// about 512 items, one round of resident workgroups -- up to four chunks.  Every
// workgroup derives the same cg from the count.  The first item's node id is read
// together with the count.
constexpr int kMaxCg = 4;  // chunks per R1 item at most
__global__ __launch_bounds__(kCThreads) void chain_hist_kernel(RejArgs a, NodeWs w) {
  __shared__ unsigned long long s_P[4][kHN], s_Q[4][kHN];  // copy (wave % 4): few lanes ever meet
  const int tid = threadIdx.x, cp = (tid >> 6) & 3;
  const int nodes = a.batch * a.n_max;
  const int act = (int)(*w.act_count);
  const int cg = min(kMaxCg, max(1, (act * a.nch + 511) / 512));
  const int ng = cg == 1 ? a.nch : (a.nch + cg - 1) / cg;  // groups per node
  const int items = act * ng;
  const int first_nd = w.act_list[min((int)blockIdx.x / ng, nodes - 1)];
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int nd = it == (int)blockIdx.x ? first_nd : w.act_list[it / ng];
    const int c_first = (it % ng) * cg, c_last = min(a.nch, c_first + cg);
    const NodeInfo inf = w.info[nd];
    const float mt = inf.mt, md = inf.md;
    const float* lt = a.tgt_logits + (int64_t)nd * a.vocab;
    const float* ld = a.dft_logits + (int64_t)nd * a.vocab;
    // the group's first chunk is in flight while the LDS histograms are cleared, and
    // each later chunk while the previous one is binned
    float xl[kCPer], xd[kCPer];
    load_chunk4(lt, c_first * kChunk, a.vocab, a.vec, xl);
    load_chunk4(ld, c_first * kChunk, a.vocab, a.vec, xd);
    for (int i = tid; i < 4 * kHN; i += blockDim.x) {
      (&s_P[0][0])[i] = 0;
      (&s_Q[0][0])[i] = 0;
    }
    __syncthreads();
    auto bin = [&](const float* bl, const float* bd) {
#pragma unroll
      for (int s2 = 0; s2 < kCPer; ++s2) {
        const float ep = exp2_arg(bl[s2], mt, a.est), eq = exp2_arg(bd[s2], md, a.esd);
        const float pp = __builtin_amdgcn_exp2f(ep), qq = __builtin_amdgcn_exp2f(eq);
        const int h = est_bucket(ep, eq, pp, qq, inf.K);
        if (h >= 0) {
          atomicAdd(&s_P[cp][h], (unsigned long long)fx42(pp));
          atomicAdd(&s_Q[cp][h], (unsigned long long)fx42(qq));
        }
      }
    };
    if (cg == 1) {
      bin(xl, xd);
    } else {
      for (int chunk = c_first; chunk < c_last; ++chunk) {
        float yl[kCPer], yd[kCPer];
        if (chunk + 1 < c_last) {
          load_chunk4(lt, (chunk + 1) * kChunk, a.vocab, a.vec, yl);
          load_chunk4(ld, (chunk + 1) * kChunk, a.vocab, a.vec, yd);
        }
        bin(xl, xd);
        if (chunk + 1 < c_last)
#pragma unroll
          for (int s2 = 0; s2 < kCPer; ++s2) {
            xl[s2] = yl[s2];
            xd[s2] = yd[s2];
          }
      }
    }
    __syncthreads();
    unsigned long long* hg = (unsigned long long*)w.hist + (int64_t)nd * 2 * kHN;
    for (int i = tid; i < kHN; i += blockDim.x) {
      const unsigned long long P = s_P[0][i] + s_P[1][i] + s_P[2][i] + s_P[3][i];
      const unsigned long long Q = s_Q[0][i] + s_Q[1][i] + s_Q[2][i] + s_Q[3][i];
      if (P) atomicAdd(&hg[2 * i], P);
      if (Q) atomicAdd(&hg[2 * i + 1], Q);
    }
    __syncthreads();  // LDS is reused by the next item
  }
}

// ---------------------------------------------------------------------------
// R2: intervals, exact sums above each interval, in-interval list, draw sums
// ---------------------------------------------------------------------------
// Levels: l = 0 .. k-1 is the threshold after l + 1 rejections, c_{l+1} in
// I_l = [a_l, b_l] (I_0 = [1, 1]); g(c) = c + W(c) is nondecreasing, so
// I_{l+1} = [a_l + lower W(a_l), b_l + upper W(b_l)], padded for rounding.  With
// H_l the first bucket certainly above b_l and G_l the first bucket that may hold
// rho > a_l:
//   P_above(l) = sum_{rho > b_l} p = S[H_l] + (tokens of buckets [G_l, H_l) with rho > b_l),
// and the tokens of [G_l, H_l) with a_l < rho <= b_l are kept in the node's list.
__global__ __launch_bounds__(kXThreads) void chain_exact_kernel(RejArgs a, NodeWs w) {
  __shared__ BucketRec s_T[kHN + 1];
  __shared__ long long s_wt[2][kXThreads / 64];
  __shared__ double s_a[kMaxKids], s_b[kMaxKids];
  __shared__ int s_G[kMaxKids], s_H[kMaxKids];
  __shared__ unsigned long long s_mask[kHN];  // levels whose edge range holds bucket h
  __shared__ unsigned long long s_EP[kMaxKids], s_EQ[kMaxKids];
  __shared__ QEntry s_q[kQueue];
  __shared__ ListEntry s_list[kWgList];
  __shared__ long long s_ll[kXThreads / 64];
  __shared__ int s_qn, s_nlist, s_base, s_bad;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
  const int nodes = a.batch * a.n_max;
  const int items = (int)(*w.act_count) * a.nch;
  const int first_nd = w.act_list[min((int)blockIdx.x / a.nch, nodes - 1)];
  fill_edges(s_T);  // ratio ranges are the same for every node
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int nd = it == (int)blockIdx.x ? first_nd : w.act_list[it / a.nch];
    const int chunk = it % a.nch;
    const NodeInfo inf = w.info[nd];
    const int k = __popcll(inf.kids);
    const float mt = inf.mt, md = inf.md;
    // merged histogram -> suffix sums S[h] = sum_{h' >= h} hist[h'], S[kHN] = 0; it is
    // loaded before the chunk's logits, which are only needed after the intervals
    // (thread t holds bucket t < kHB; the kHN - kHB top buckets are added to every suffix)
    const long long* hg = w.hist + (int64_t)nd * 2 * kHN;
    const long long v0 = hg[2 * tid], v1 = hg[2 * tid + 1];
    long long tp[kHN - kHB], tq[kHN - kHB];
#pragma unroll
    for (int j = 0; j < kHN - kHB; ++j) {
      tp[j] = hg[2 * (kHB + j)];
      tq[j] = hg[2 * (kHB + j) + 1];
    }
    float xl[kXPer], xd[kXPer];
    load_chunk8(a.tgt_logits + (int64_t)nd * a.vocab, chunk * kChunk, a.vocab, a.vec, xl);
    load_chunk8(a.dft_logits + (int64_t)nd * a.vocab, chunk * kChunk, a.vocab, a.vec, xd);
    for (int l = tid; l < k; l += blockDim.x) s_EP[l] = s_EQ[l] = 0;
    for (int h = tid; h < kHN; h += blockDim.x) s_mask[h] = 0;
    if (tid == 0) {
      s_qn = 0;
      s_nlist = 0;
      s_bad = 0;
    }
    {
      // suffix within the wave = wave total - inclusive prefix + own value
      const long long p0 = wave_incl_scan_ll(v0), p1 = wave_incl_scan_ll(v1);
      const long long w0 = lane63_ll(p0), w1 = lane63_ll(p1);
      long long i0 = w0 - p0 + v0, i1 = w1 - p1 + v1;
      if (lane == 0) {
        s_wt[0][wv] = w0;
        s_wt[1][wv] = w1;
      }
      __syncthreads();
      for (int x = wv + 1; x < nw; ++x) {
        i0 += s_wt[0][x];
        i1 += s_wt[1][x];
      }
      long long top0 = 0, top1 = 0;  // suffix sums of the top buckets
#pragma unroll
      for (int j = kHN - kHB - 1; j >= 0; --j) {
        top0 += tp[j];
        top1 += tq[j];
        if (tid == j) {
          s_T[kHB + j].SP = top0;
          s_T[kHB + j].SQ = top1;
        }
      }
      s_T[tid].SP = i0 + top0;
      s_T[tid].SQ = i1 + top1;
      if (tid == 0) {
        s_T[kHN].SP = 0;
        s_T[kHN].SQ = 0;
      }
    }
    __syncthreads();
    // interval chains: lower ends on wavefront 0, upper ends on wavefront 1, each
    // level's bound evaluated by the whole wavefront
    if (wv == 0) {
      double c = 1.0;
      if (lane == 0) s_a[0] = 1.0;
      for (int l = 1; l < k; ++l) {
        const double na = c + w_bound_wave(c, s_T, inf.izt, inf.izd, false);
        c = na - 1e-10 * na;
        if (lane == 0) s_a[l] = c;
      }
    } else if (wv == 1) {
      double c = 1.0;
      if (lane == 0) s_b[0] = 1.0;
      for (int l = 1; l < k; ++l) {
        const double nb = c + w_bound_wave(c, s_T, inf.izt, inf.izd, true);
        c = nb + 1e-10 * nb;
        if (lane == 0) s_b[l] = c;
        if (!(c < 15.5)) {  // beyond the histogram: direct path
          if (lane == 0) {
            s_bad = 1;
            for (int m = l + 1; m < k; ++m) s_b[m] = c;
          }
          break;
        }
      }
    }
    __syncthreads();
    for (int l = tid; l < k; l += blockDim.x) {
      const int G = first_maybe(s_a[l], s_T), H = s_bad ? kHN : first_above(s_b[l], s_T);
      s_G[l] = G;
      s_H[l] = H;
      if (H > kHTop || H - G > kMaxEdge) s_bad = 1;
    }
    __syncthreads();
    if (s_bad) {
      if (chunk == 0 && tid == 0) atomicOr(&w.rec[nd].flags, kFlagFallback);
      __syncthreads();
      continue;
    }
    for (int x = tid; x < k * kMaxEdge; x += blockDim.x) {  // mark the edge ranges
      const int l = x / kMaxEdge, h = s_G[l] + x % kMaxEdge;
      if (h < s_H[l]) atomicOr(&s_mask[h], 1ull << l);
    }
    if (chunk == 0) {  // the certain part above each interval, and the intervals
      unsigned long long* lv = (unsigned long long*)w.lvl + (int64_t)nd * 2 * kMaxKids;
      for (int l = tid; l < k; l += blockDim.x) {
        const int H = s_H[l];
        if (s_T[H].SP) atomicAdd(&lv[2 * l], (unsigned long long)s_T[H].SP);
        if (s_T[H].SQ) atomicAdd(&lv[2 * l + 1], (unsigned long long)s_T[H].SQ);
        w.rec[nd].a[l] = s_a[l];
        w.rec[nd].b[l] = s_b[l];
      }
    }
    __syncthreads();
    const int htop = s_H[k - 1];
    long long cp = 0, cq = 0;  // this chunk's tokens with rho > b_{k-1} (the terminal draw)
    int hh[kXPer];
    float pq[kXPer], qq2[kXPer];
    unsigned edge = 0;
#pragma unroll
    for (int s2 = 0; s2 < kXPer; ++s2) {
      const float ep = exp2_arg(xl[s2], mt, a.est), eq = exp2_arg(xd[s2], md, a.esd);
      const float pp = __builtin_amdgcn_exp2f(ep), qq = __builtin_amdgcn_exp2f(eq);
      const int h = est_bucket(ep, eq, pp, qq, inf.K);
      const bool above = h >= htop;
      cp += above ? fx42(pp) : 0;
      cq += above ? fx42(qq) : 0;
      hh[s2] = h;
      pq[s2] = pp;
      qq2[s2] = qq;
    }
#pragma unroll
    for (int s2 = 0; s2 < kXPer; ++s2) {
      const int h = hh[s2];
      if (h >= 0 && h < htop && s_mask[h]) edge |= 1u << s2;
    }
    // queue slots: one LDS atomic per wavefront
    const int ne = __popc(edge);
    const int pre = wave_incl_scan_i(ne);
    int qbase = 0;
    if (lane == 63 && pre) qbase = atomicAdd(&s_qn, pre);
    qbase = lane63_i(qbase) + pre - ne;
#pragma unroll
    for (int s2 = 0; s2 < kXPer; ++s2) {
      if (edge & (1u << s2)) {
        if (qbase < kQueue) s_q[qbase] = QEntry{xtok(chunk * kChunk, s2), hh[s2], pq[s2], qq2[s2]};
        ++qbase;
      }
    }
    __syncthreads();
    const int qn = s_qn;
    const double btop = s_b[k - 1];
    for (int i = tid; i < min(qn, kQueue); i += blockDim.x) {
      const QEntry e = s_q[i];
      const double p = (double)e.pp * inf.izt, q = (double)e.qq * inf.izd;
      const double rho = q > 0.0 ? p / q : INFINITY;
      const long long fp = fx42(e.pp), fq = fx42(e.qq);
      if (rho > btop) {
        cp += fp;
        cq += fq;
      }
      bool in_list = false;
      for (unsigned long long m = s_mask[e.h]; m; m &= m - 1) {
        const int l = __ffsll(m) - 1;
        if (rho > s_b[l]) {
          if (fp) atomicAdd(&s_EP[l], (unsigned long long)fp);
          if (fq) atomicAdd(&s_EQ[l], (unsigned long long)fq);
        } else if (rho > s_a[l]) {
          in_list = true;
        }
      }
      if (in_list) {
        const int x = atomicAdd(&s_nlist, 1);
        if (x < kWgList) s_list[x] = ListEntry{fp, fq, rho, e.tok, 0};
      }
    }
    cp = block_sum_ll(cp, s_ll);
    cq = block_sum_ll(cq, s_ll);
    if (tid == 0) {
      long long* cd = w.cdraw + ((int64_t)nd * a.nch + chunk) * 2;
      cd[0] = cp;
      cd[1] = cq;
      const int n_in = s_nlist;
      if (qn > kQueue || n_in > kWgList) {
        atomicOr(&w.rec[nd].flags, kFlagFallback);
        s_base = -1;
      } else {
        s_base = n_in ? (int)atomicAdd(&w.list_n[nd], (uint32_t)n_in) : 0;
        if (s_base + n_in > kListCap) atomicOr(&w.rec[nd].flags, kFlagFallback);
      }
    }
    unsigned long long* lv = (unsigned long long*)w.lvl + (int64_t)nd * 2 * kMaxKids;
    for (int l = tid; l < k; l += blockDim.x) {
      if (s_EP[l]) atomicAdd(&lv[2 * l], s_EP[l]);
      if (s_EQ[l]) atomicAdd(&lv[2 * l + 1], s_EQ[l]);
    }
    __syncthreads();
    const int n_in = min(s_nlist, kWgList);
    if (s_base >= 0)
      for (int i = tid; i < n_in; i += blockDim.x)
        if (s_base + i < kListCap) w.list[(int64_t)nd * kListCap + s_base + i] = s_list[i];
    __syncthreads();  // LDS is reused by the next item
  }
}

// ---------------------------------------------------------------------------
// R3: every node, then the walk
// ---------------------------------------------------------------------------
// w(t) = max(0, p - c q); c == 0 is p itself.
__device__ inline double resid_el(const RejArgs& a, const RowView& r, int t, double c) {
  const double p = p_el(a, r, r.lt[t]);
  if (c == 0.0) return p;
  return fmax(0.0, p - c * q_el(a, r, r.ld[t]));
}

// Direct W(c) over the whole vocabulary.
__device__ double direct_W(const RejArgs& a, const RowView& r, double c, double* s_red) {
  double acc = 0.0;
  for (int t = threadIdx.x; t < a.vocab; t += blockDim.x) acc += resid_el(a, r, t, c);
  return block_sum_d(acc, s_red);
}

// Inverse-CDF search inside tokens [t0, t1): the smallest t whose running sum,
// added to `pre`, exceeds `target`.  Each thread owns a contiguous run; runs are
// combined by an exclusive scan in thread order.  Returns -1 if rounding leaves no
// crossing in the range.  elem(t) gives the unnormalised mass of token t.
template <typename Elem>
__device__ int scan_range(int t0, int t1, double pre, double target, Elem elem, double* s_w, int* s_pick) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (t1 - t0 + nt - 1) / nt;
  const int r0 = t0 + tid * per, r1 = min(t1, r0 + per);
  double own = 0.0;
  for (int t = r0; t < r1; ++t) own += elem(t);
  if (tid == 0) *s_pick = 0x7fffffff;
  double total;
  const double before = pre + block_excl_scan_d(own, s_w, &total);
  if (r0 < r1 && before + own > target && !(before > target)) {
    double run = 0.0;
    int pick = r1 - 1;
    for (int t = r0; t < r1; ++t) {
      run += elem(t);
      if (before + run > target) {
        pick = t;
        break;
      }
    }
    atomicMin(s_pick, pick);  // rounding may let two adjacent runs both claim it
  }
  __syncthreads();
  const int k = *s_pick == 0x7fffffff ? -1 : *s_pick;
  __syncthreads();
  return k;
}

// Largest token in [t0, t1) with positive mass (rounding fallback), or -1.
template <typename Elem>
__device__ int last_positive(int t0, int t1, Elem elem, int* s_pick) {
  int best = -1;
  for (int t = t0 + threadIdx.x; t < t1; t += blockDim.x)
    if (elem(t) > 0.0) best = t;
  best = wave_max_i(best);
  __syncthreads();
  if (threadIdx.x == 0) *s_pick = -1;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) atomicMax(s_pick, best);
  __syncthreads();
  const int k = *s_pick;
  __syncthreads();
  return k;
}

// Inverse-CDF search inside one chunk [t0, t1) with a 256-thread block: thread i owns
// the contiguous run t0 + i * kPer .. + kPer - 1, held in registers.  Masses are
// exp((l - mc)/T) * scale for a leaf (the softmax chunk partial's reference mc), or
// max(0, p - c q) for a residual.  Returns the smallest token whose running sum
// added to `pre` exceeds `target`, or -1 if rounding leaves no crossing.
__device__ int chunk_scan(const RejArgs& a, const RowView& rv, int t0, int t1, bool resid, float mc, double scale,
                          double c, double pre, double target, double* s_w, int* s_pick) {
  const int tid = threadIdx.x;
  const int r0 = t0 + tid * kPer;
  float xl[kPer], xd[kPer];
  load_run(rv.lt, r0, t1, a.vec, xl);
  if (resid) load_run(rv.ld, r0, t1, a.vec, xd);
  auto mass = [&](int s2) -> double {
    if (!resid) return (double)exp_scaled(xl[s2] - mc, a.est) * scale;
    return fmax(0.0, p_el(a, rv, xl[s2]) - c * q_el(a, rv, xd[s2]));
  };
  double own = 0.0;
#pragma unroll
  for (int s2 = 0; s2 < kPer; ++s2) own += mass(s2);
  if (tid == 0) *s_pick = 0x7fffffff;
  double total;
  const double before = pre + block_excl_scan_d(own, s_w, &total);
  if (r0 < t1 && before + own > target && !(before > target)) {
    double run = 0.0;
    int pick = min(t1, r0 + kPer) - 1;
#pragma unroll
    for (int s2 = 0; s2 < kPer; ++s2) {
      run += mass(s2);
      if (before + run > target) {
        pick = r0 + s2;
        break;
      }
    }
    atomicMin(s_pick, pick);
  }
  __syncthreads();
  const int k = *s_pick == 0x7fffffff ? -1 : *s_pick;
  __syncthreads();
  return k;
}

// Direct inverse-CDF draw over the whole vocabulary, in kChunk pieces.
__device__ int direct_draw(const RejArgs& a, const RowView& r, double c, double u, double* s_red, double* s_w,
                           int* s_pick) {
  const int nch = (a.vocab + kChunk - 1) / kChunk;
  auto el = [&](int t) { return resid_el(a, r, t, c); };
  // chunk totals in chunk order (each one a fixed-order block reduction)
  double S = 0.0;
  for (int ch = 0; ch < nch; ++ch) {
    double acc = 0.0;
    const int t0 = ch * kChunk, t1 = min(a.vocab, t0 + kChunk);
    for (int t = t0 + threadIdx.x; t < t1; t += blockDim.x) acc += el(t);
    S += block_sum_d(acc, s_red);
  }
  if (!(S > 0.0)) return -1;
  const double target = u * S;
  double pre = 0.0;
  for (int ch = 0; ch < nch; ++ch) {
    double acc = 0.0;
    const int t0 = ch * kChunk, t1 = min(a.vocab, t0 + kChunk);
    for (int t = t0 + threadIdx.x; t < t1; t += blockDim.x) acc += el(t);
    const double sc = block_sum_d(acc, s_red);
    if (pre + sc > target || ch == nch - 1) {
      int k = scan_range(t0, t1, pre, target, el, s_w, s_pick);
      if (k < 0) k = last_positive(0, a.vocab, el, s_pick);
      return k;
    }
    pre += sc;
  }
  return -1;
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

// One workgroup per node slot.  Node results go to the workspace; the request's
// last workgroup walks from the root and writes accepted_child / term_token.
struct SibState {
  uint64_t rest;  // children not yet tested
  double c, W;
  int acc, lvl, zero_last, pending;  // pending: a rejection whose W needs a direct pass
};
__global__ __launch_bounds__(kRjThreads) void node_kernel(RejArgs a, NodeWs w, int chunked) {
  __shared__ float s_ua[64];
  __shared__ double s_px[64], s_qx[64];
  __shared__ long long s_lv[2 * kMaxKids];
  __shared__ double s_ia[kMaxKids], s_ib[kMaxKids];
  __shared__ ListEntry s_list[kLdsList];
  __shared__ double s_red[kRjThreads / 64];
  __shared__ double s_w[8];
  __shared__ double s_chunk[256];
  __shared__ float s_cmx[256];
  __shared__ unsigned long long s_cP[256], s_cQ[256];
  __shared__ int s_pick, s_flags, s_nlist, s_last;
  __shared__ SibState s_st;
  __shared__ NodeRes s_res[64];
  __shared__ int s_oacc[64], s_oterm[64], s_tok[64], s_pn[64], s_ot[64], s_len;
  const int tid = threadIdx.x, lane = tid & 63;
  const int nd = blockIdx.x;
  const int b = nd / a.n_max, n = nd % a.n_max;
  const int64_t base = (int64_t)b * a.n_max, row = nd;
  if (blockIdx.x == 0 && tid == 0 && chunked) *w.act_count = 0;  // R1 and R2 are done with it
  // ---- everything this node may need, in one round of loads: its plan record,
  // and (chunked vocabularies) the chain state R2 left for it, which is valid
  // memory for every node slot and kept only if the node turns out to need it ----
  const NodeInfo inf = w.info[nd];
  static_assert(kMaxKids <= kRjThreads && 2 * kMaxKids <= kRjThreads && kLdsList % kRjThreads == 0, "R3 preload");
  double sp_a = 0.0, sp_b = 0.0;
  long long sp_lv = 0, sp_cp = 0, sp_cq = 0;
  int sp_flags = 0;
  uint32_t sp_n = 0;
  constexpr int kSpE = kLdsList / kRjThreads;  // list entries per thread
  long long sp_fp[kSpE] = {}, sp_fq[kSpE] = {};
  double sp_rho[kSpE] = {};
  int sp_tok[kSpE] = {};
  if (chunked) {
    const ChainRec* R = w.rec + nd;
    if (tid < kMaxKids) {
      sp_a = R->a[tid];
      sp_b = R->b[tid];
    }
    if (tid < 2 * kMaxKids) sp_lv = w.lvl[(int64_t)nd * 2 * kMaxKids + tid];
    if (tid < a.nch) {
      const long long* cd = w.cdraw + (int64_t)nd * a.nch * 2;
      sp_cp = cd[2 * tid];
      sp_cq = cd[2 * tid + 1];
    }
    sp_flags = R->flags;
    sp_n = w.list_n[nd];
    const ListEntry* L0 = w.list + (int64_t)nd * kListCap;
#pragma unroll
    for (int j = 0; j < kSpE; ++j) {
      const ListEntry* e = L0 + tid + kRjThreads * j;
      sp_fp[j] = e->fp;
      sp_fq[j] = e->fq;
      sp_rho[j] = e->rho;
      sp_tok[j] = e->tok;
    }
  }
  const int nb = a.n_nodes[b];
  if (tid < 64) {
    const bool in = tid < a.n_max;
    s_ua[tid] = in ? a.u_accept[base + tid] : 0.0f;
    const KidInfo ki = in ? w.kid[base + tid] : KidInfo{0.0, 0.0};
    s_px[tid] = ki.px;
    s_qx[tid] = ki.qx;
  }
  RowView rv;
  rv.lt = a.tgt_logits + row * (int64_t)a.vocab;
  rv.ld = a.dft_logits + row * (int64_t)a.vocab;
  rv.mt = inf.mt;
  rv.md = inf.md;
  rv.izt = inf.izt;
  rv.izd = inf.izd;
  const float us = a.u_sample[row];
  const int k = __popcll(inf.kids);
  const bool node_ok = inf.verdict == 0 && n < nb;
  const bool chain = chunked && node_ok && inf.active;
  if (chain) {  // (loaded above in the first round; kept only for chain nodes)
    const int nl = (int)min(sp_n, (uint32_t)kListCap);
    if (tid < k) {
      s_ia[tid] = sp_a;
      s_ib[tid] = sp_b;
    }
    if (tid < 2 * k) s_lv[tid] = sp_lv;
    if (tid < a.nch) {
      s_cP[tid] = (unsigned long long)sp_cp;
      s_cQ[tid] = (unsigned long long)sp_cq;
    }
#pragma unroll
    for (int j = 0; j < kSpE; ++j)
      if (nl <= kLdsList && tid + kRjThreads * j < nl)
        s_list[tid + kRjThreads * j] = ListEntry{sp_fp[j], sp_fq[j], sp_rho[j], sp_tok[j], 0};
    if (tid == 0) {
      s_flags = sp_flags;
      s_nlist = nl;
    }
  }
  const bool leaf_chunks = chunked && node_ok && k == 0 && a.tgt_chunk_max != nullptr;
  if (leaf_chunks && tid < a.nch) {
    const float cm = a.tgt_chunk_max[row * a.nch + tid];
    s_cmx[tid] = cm;
    s_chunk[tid] = a.tgt_chunk_sum[row * a.nch + tid] * exp(((double)cm - (double)rv.mt) * a.inv_t);
  }
  __syncthreads();
  NodeRes res{SPEC_NODE_NOT_EVALUATED, SPEC_NODE_NOT_EVALUATED, 0, 0};
  bool used_direct = false;  // a direct vocabulary pass (counted for multi-chunk vocabularies)
  if (node_ok) {
    if (isnan(rv.mt) || isnan(rv.md)) {
      res.err = 1;
    } else {
      int acc = SPEC_NODE_NONE, term = -1;
      if (k == 0) {
        // ---- leaf: the bonus is drawn from p ----
        const double u = (double)us;
        if (leaf_chunks) {
          double pre, target;
          const int ch = pick_chunk(s_chunk, a.nch, u, s_w, &s_pick, &pre, &target);
          const float mc = s_cmx[ch];
          const double scale = exp(((double)mc - (double)rv.mt) * a.inv_t);
          const int t0 = ch * kChunk, t1 = min(a.vocab, t0 + kChunk);
          term = chunk_scan(a, rv, t0, t1, false, mc, scale, 0.0, pre, target, s_w, &s_pick);
          if (term < 0) {
            auto el = [&](int t) { return (double)exp_scaled(rv.lt[t] - mc, a.est) * scale; };
            term = last_positive(t0, t1, el, &s_pick);
          }
        } else {
          term = direct_draw(a, rv, 0.0, u, s_red, s_w, &s_pick);
        }
      } else {
        // ---- children in ascending index, tested against the running residual ----
        const bool fast = chain && !(s_flags & kFlagFallback);
        const ListEntry* L = w.list + (int64_t)nd * kListCap;
        const int nlist = fast ? s_nlist : 0;
        const bool in_lds = nlist <= kLdsList;  // then s_list holds it (filled with the preload)
        const ListEntry* LL = in_lds ? s_list : L;
        if (tid == 0) s_st = SibState{inf.kids, 0.0, 1.0, SPEC_NODE_NONE, 0, 0, 0};
        __syncthreads();
        // A short list (the usual case): wavefront 0 follows the exact path with the
        // level data in registers, lane l holding level l (its child's test inputs,
        // interval and exact sums above it) and lane i list entry i; each level
        // fetches what it needs with readlane, and the listed tokens inside the
        // interval come from one ballot.  The sums are exact integers, so the
        // result equals the wavefront version below.
        if (fast && nlist <= kShortList && tid < 64) {
          const int kk = min(k, 64);
          uint64_t rest_l = inf.kids;  // children left after the child of level `lane`
          for (int i = 0; i < lane && rest_l; ++i) rest_l &= rest_l - 1;
          const int ci_l = rest_l ? __ffsll((unsigned long long)rest_l) - 1 : 0;
          rest_l = rest_l ? rest_l & (rest_l - 1) : 0;
          const bool lv_in = lane < kk;
          const float u_l = lv_in ? s_ua[ci_l] : 0.0f;
          const double px_l = lv_in ? s_px[ci_l] : 0.0, qx_l = lv_in ? s_qx[ci_l] : 0.0;
          const double ia_l = lv_in ? s_ia[lane] : 0.0, ib_l = lv_in ? s_ib[lane] : 0.0;
          const long long lp_l = lv_in ? s_lv[2 * lane] : 0, lq_l = lv_in ? s_lv[2 * lane + 1] : 0;
          const bool e_in = lane < nlist;
          const double er_l = e_in ? s_list[lane].rho : -1.0;
          const long long ep_l = e_in ? s_list[lane].fp : 0, eq_l = e_in ? s_list[lane].fq : 0;
          auto rl_i = [](int v, int l) { return __builtin_amdgcn_readlane(v, l); };
          auto rl_ll = [&](long long v, int l) {
            return (long long)(((unsigned long long)(uint32_t)rl_i((int)(v >> 32), l) << 32) |
                               (uint32_t)rl_i((int)(uint32_t)v, l));
          };
          auto rl_d = [&](double v, int l) { return __longlong_as_double(rl_ll(__double_as_longlong(v), l)); };
          // The thresholds depend only on earlier rejections, not on the tests'
          // outcomes, so the serial pass carries the (c, W) recursion alone, for every
          // level, and lane l keeps the state child l is tested with; the tests then
          // run in parallel and the first accepted level wins.  The same arithmetic as
          // testing level by level, without the division on the serial path.
          double c = 0.0, W = 1.0;
          int zl = 0, pend_at = kk;  // pend_at: the first transition that leaves its interval
          double c_my = 0.0, W_my = 1.0;
          for (int l = 0; l < kk; ++l) {
            if (lane == l) {
              c_my = c;
              W_my = W;
            }
            const double cn = c + W;  // the threshold after a rejection at this level
            const double ia = rl_d(ia_l, l), ib = rl_d(ib_l, l);
            if (!(cn >= ia && cn <= ib)) {
              pend_at = l;
              break;
            }
            long long lp = rl_ll(lp_l, l), lq = rl_ll(lq_l, l);
            for (uint64_t bits = __ballot(e_in && er_l > cn && er_l <= ib); bits; bits &= bits - 1) {
              const int j = __ffsll((unsigned long long)bits) - 1;
              lp += rl_ll(ep_l, j);
              lq += rl_ll(eq_l, j);
            }
            const double Wn = ((double)lp * rv.izt - cn * (double)lq * rv.izd) * kFxInv;
            if (Wn > 0.0) {
              c = cn;
              W = Wn;
              zl = 0;
            } else {
              zl = 1;  // the residual keeps its previous threshold
            }
          }
          // levels 0 .. min(kk, pend_at + 1) - 1 have their test inputs
          const bool ok = lane < min(kk, pend_at + 1) && (double)u_l < accept_ratio(px_l, qx_l, c_my, W_my);
          const uint64_t okm = __ballot(ok);
          int acc0 = SPEC_NODE_NONE, lvl, pend = 0;
          uint64_t m;
          if (okm) {  // the first accepted level (the state is not used after an acceptance)
            const int l = __ffsll((unsigned long long)okm) - 1;
            acc0 = rl_i(ci_l, l);
            lvl = l;
            m = (uint64_t)rl_ll((long long)rest_l, l);
          } else if (pend_at < kk) {  // every tested child rejected, then a transition to finish directly
            lvl = pend_at + 1;
            pend = 1;
            m = (uint64_t)rl_ll((long long)rest_l, pend_at);
          } else {  // every child rejected
            lvl = kk;
            m = (uint64_t)rl_ll((long long)rest_l, kk - 1);
          }
          if (lane == 0) s_st = SibState{m, c, W, acc0, lvl, zl, pend};
        }
        // otherwise wavefront 0 follows it, the list spread over its lanes
        if (fast && nlist > kShortList && tid < 64) {
          // this lane's list entries stay in registers across the levels
          double er[kLdsList / 64];
          long long efp[kLdsList / 64], efq[kLdsList / 64];
#pragma unroll
          for (int j = 0; j < kLdsList / 64; ++j) {
            const int i = lane + 64 * j;
            er[j] = -1.0;  // never above a threshold
            efp[j] = efq[j] = 0;
            if (in_lds && i < nlist) {
              const ListEntry e = s_list[i];
              er[j] = e.rho;
              efp[j] = e.fp;
              efq[j] = e.fq;
            }
          }
          uint64_t m = inf.kids;
          double c = 0.0, W = 1.0;
          int acc0 = SPEC_NODE_NONE, lvl = 0, zl = 0, pend = 0;
          while (m) {
            const int ci = __ffsll((unsigned long long)m) - 1;
            m &= m - 1;
            if ((double)s_ua[ci] < accept_ratio(s_px[ci], s_qx[ci], c, W)) {
              acc0 = ci;
              break;
            }
            ++lvl;  // cn = c + W is the threshold after this rejection
            const double cn = c + W;
            const double ia = s_ia[lvl - 1], ib = s_ib[lvl - 1];
            if (!(cn >= ia && cn <= ib)) {
              pend = 1;
              break;
            }
            long long lp = 0, lq = 0;  // listed tokens inside the interval and above cn
            if (in_lds) {
#pragma unroll
              for (int j = 0; j < kLdsList / 64; ++j) {
                const bool inside = er[j] > cn && er[j] <= ib;
                lp += inside ? efp[j] : 0;
                lq += inside ? efq[j] : 0;
              }
            } else {
              for (int i = lane; i < nlist; i += 64) {
                const ListEntry e = LL[i];
                if (e.rho > cn && e.rho <= ib) {
                  lp += e.fp;
                  lq += e.fq;
                }
              }
            }
            lp = wave_sum_ll(lp);
            lq = wave_sum_ll(lq);
            const double Wn =
                ((double)(s_lv[2 * (lvl - 1)] + lp) * rv.izt - cn * (double)(s_lv[2 * (lvl - 1) + 1] + lq) * rv.izd) *
                kFxInv;
            if (Wn > 0.0) {
              c = cn;
              W = Wn;
              zl = 0;
            } else {
              zl = 1;  // the residual keeps its previous threshold
            }
          }
          if (lane == 0) s_st = SibState{m, c, W, acc0, lvl, zl, pend};
        }
        __syncthreads();
        const SibState st = s_st;
        __syncthreads();
        acc = st.acc;
        double c = st.c, W = st.W;
        bool zero_last = st.zero_last;
        const bool fell_back = !fast || st.pending;
        if (acc < 0 && fell_back) {  // finish with direct vocabulary passes
          if (st.pending) {
            const double cn = c + W;
            const double Wn = direct_W(a, rv, cn, s_red);
            used_direct = true;
            if (Wn > 0.0) {
              c = cn;
              W = Wn;
              zero_last = false;
            } else {
              zero_last = true;
            }
          }
          for (uint64_t m = st.rest; m; m &= m - 1) {
            const int ci = __ffsll((unsigned long long)m) - 1;
            if ((double)s_ua[ci] < accept_ratio(s_px[ci], s_qx[ci], c, W)) {
              acc = ci;
              break;
            }
            const double cn = c + W;
            const double Wn = direct_W(a, rv, cn, s_red);
            used_direct = true;
            if (Wn > 0.0) {
              c = cn;
              W = Wn;
              zero_last = false;
            } else {
              zero_last = true;
            }
          }
        }
        if (acc < 0) {
          // ---- all children rejected: the bonus is drawn from the residual ----
          const double u = (double)us;
          if (!fell_back && !zero_last) {
            const double ib = s_ib[k - 1];
            for (int i = tid; i < nlist; i += blockDim.x) {
              const ListEntry e = LL[i];
              if (e.rho > c && e.rho <= ib) {
                const int ch = e.tok / kChunk;
                atomicAdd(&s_cP[ch], (unsigned long long)e.fp);
                atomicAdd(&s_cQ[ch], (unsigned long long)e.fq);
              }
            }
            __syncthreads();
            if (tid < a.nch)
              s_chunk[tid] = ((double)(long long)s_cP[tid] * rv.izt - c * (double)(long long)s_cQ[tid] * rv.izd) * kFxInv;
            __syncthreads();
            double pre, target;
            const int ch = pick_chunk(s_chunk, a.nch, u, s_w, &s_pick, &pre, &target);
            const int t0 = ch * kChunk, t1 = min(a.vocab, t0 + kChunk);
            term = chunk_scan(a, rv, t0, t1, true, 0.0f, 1.0, c, pre, target, s_w, &s_pick);
            if (term < 0) {
              const double cc = c;
              auto el = [&](int t) { return resid_el(a, rv, t, cc); };
              term = last_positive(t0, t1, el, &s_pick);
            }
          } else {
            term = direct_draw(a, rv, c, u, s_red, s_w, &s_pick);
            used_direct = true;
          }
        }
      }
      res.acc = acc;
      res.term = acc >= 0 ? SPEC_NODE_NOT_EVALUATED : term;
    }
  }
  if (used_direct && chunked && tid == 0) atomicAdd(&w.diag[kDiagDirect], 1u);
  if (chain) {  // the chain state of this node is consumed: clear it for the next call
    __syncthreads();
    long long* hw = w.hist + (int64_t)nd * 2 * kHN;
    for (int i = tid; i < 2 * kHN; i += blockDim.x) hw[i] = 0;
    for (int i = tid; i < 2 * kMaxKids; i += blockDim.x) w.lvl[(int64_t)nd * 2 * kMaxKids + i] = 0;
    if (tid == 0) {
      w.list_n[nd] = 0;
      w.rec[nd].flags = 0;
    }
  }
  // ---- publish; the request's last workgroup walks ----
  if (tid == 0) {
    pub_store(&w.res[nd].acc, res.acc);
    pub_store(&w.res[nd].term, res.term);
    pub_store(&w.res[nd].err, res.err);
    stores_done();
    s_last = pub_arrive(&w.req_count[b]) == (uint32_t)(a.n_max - 1);
  }
  __syncthreads();
  if (!s_last) return;
  if (tid < a.n_max) {
    s_res[tid].acc = pub_load(&w.res[base + tid].acc);
    s_res[tid].term = pub_load(&w.res[base + tid].term);
    s_res[tid].err = pub_load(&w.res[base + tid].err);
    s_tok[tid] = a.path_nodes ? a.tokens[base + tid] : 0;
  }
  if (tid < 64) {
    s_oacc[tid] = SPEC_NODE_NOT_EVALUATED;
    s_oterm[tid] = SPEC_NODE_NOT_EVALUATED;
  }
  __syncthreads();
  if (tid == 0) {
    pub_store(&w.req_count[b], 0u);
    int verdict = inf.verdict;
    int cur = 0;
    for (int step = 0; verdict == 0 && step < nb; ++step) {
      const NodeRes r = s_res[cur];
      if (r.err) {
        verdict = SPEC_ERR_BAD_INPUT;
        break;
      }
      s_oacc[cur] = r.acc;
      if (r.acc >= 0) {
        cur = r.acc;
        continue;
      }
      s_oterm[cur] = r.term;
      if (r.term < 0) report(a.status, SPEC_ERR_BAD_INPUT);
      break;
    }
    if (verdict != 0) {
      for (int i = 0; i < 64; ++i) s_oacc[i] = s_oterm[i] = SPEC_NODE_NOT_EVALUATED;
      s_oacc[0] = SPEC_NODE_BAD_REQUEST;
      report(a.status, verdict);
    }
  }
  __syncthreads();
  if (tid < a.n_max) {
    a.accepted_child[base + tid] = s_oacc[tid];
    a.term_token[base + tid] = s_oterm[tid];
  }
  emit_path(a, b, s_oacc, s_oterm, s_tok, nb, s_pn, s_ot, &s_len);
}

// T == 0: one wavefront per request follows the target argmax.
__global__ __launch_bounds__(64) void greedy_walk_kernel(RejArgs a) {
  __shared__ int s_par[64], s_tok[64], s_arg[64], s_oacc[64], s_oterm[64], s_pn[64], s_ot[64];
  __shared__ float s_max[64];
  __shared__ int s_bad, s_len;
  const int tid = threadIdx.x, b = blockIdx.x;
  const int64_t base = (int64_t)b * a.n_max;
  const int nb = a.n_nodes[b];
  const bool n_ok = nb >= 1 && nb <= a.n_max;
  const bool in = tid < a.n_max;
  s_par[tid] = in ? a.parent[base + tid] : -2;
  s_tok[tid] = in ? a.tokens[base + tid] : 0;
  s_arg[tid] = in ? a.tgt_argmax[base + tid] : -1;
  s_max[tid] = in ? a.tgt_max[base + tid] : 0.0f;
  s_oacc[tid] = s_oterm[tid] = SPEC_NODE_NOT_EVALUATED;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (n_ok && tid < nb) {
    const int p = s_par[tid];
    if (tid == 0 ? p != -1 : (p < 0 || p >= tid)) atomicOr(&s_bad, 1);
    else if (tid > 0 && (s_tok[tid] < 0 || s_tok[tid] >= a.vocab)) atomicOr(&s_bad, 2);
  }
  __syncthreads();
  if (tid == 0) {
    int verdict = !n_ok || (s_bad & 1) ? SPEC_ERR_BAD_TREE : (s_bad ? SPEC_ERR_BAD_INPUT : 0);
    int cur = 0;
    for (int step = 0; verdict == 0 && step < nb; ++step) {
      if (isnan(s_max[cur])) {
        verdict = SPEC_ERR_BAD_INPUT;
        break;
      }
      const int am = s_arg[cur];
      int acc = SPEC_NODE_NONE;
      for (int c = cur + 1; c < nb; ++c)
        if (s_par[c] == cur && s_tok[c] == am) {
          acc = c;
          break;
        }
      s_oacc[cur] = acc;
      if (acc >= 0) {
        cur = acc;
        continue;
      }
      s_oterm[cur] = am;
      break;
    }
    if (verdict != 0) {
      for (int i = 0; i < 64; ++i) s_oacc[i] = s_oterm[i] = SPEC_NODE_NOT_EVALUATED;
      s_oacc[0] = SPEC_NODE_BAD_REQUEST;
      report(a.status, verdict);
    }
  }
  __syncthreads();
  if (in) {
    a.accepted_child[base + tid] = s_oacc[tid];
    a.term_token[base + tid] = s_oterm[tid];
  }
  emit_path(a, b, s_oacc, s_oterm, s_tok, nb, s_pn, s_ot, &s_len);
}

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout: node results, plan and request counters always; the chain
// arrays when the vocabulary spans two or more chunks.
inline size_t node_ws_layout(int64_t batch, int64_t nodes, int nch, char* base, NodeWs* w) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += a256(bytes);
    return p;
  };
  NodeWs t{};
  t.diag = (uint32_t*)take(16);
  t.res = (NodeRes*)take((size_t)nodes * sizeof(NodeRes));
  t.req_count = (uint32_t*)take((size_t)batch * 4);
  t.info = (NodeInfo*)take((size_t)nodes * sizeof(NodeInfo));
  t.kid = (KidInfo*)take((size_t)nodes * sizeof(KidInfo));
  if (nch >= 2) {
    t.act_count = (uint32_t*)take(4);
    t.act_list = (int32_t*)take((size_t)nodes * 4);
    t.hist = (long long*)take((size_t)nodes * kHN * 16);
    t.rec = (ChainRec*)take((size_t)nodes * sizeof(ChainRec));
    t.lvl = (long long*)take((size_t)nodes * kMaxKids * 16);
    t.cdraw = (long long*)take((size_t)nodes * nch * 16);
    t.list = (ListEntry*)take((size_t)nodes * kListCap * sizeof(ListEntry));
    t.list_n = (uint32_t*)take((size_t)nodes * 4);
  }
  if (w) *w = t;
  return off;
}

}  // namespace spectree

extern "C" size_t spec_tree_reject_sample_workspace_size(int32_t batch, int32_t n_max, int32_t vocab) {
  using namespace spectree;
  if (batch < 1 || n_max < 1 || n_max > 64 || vocab < 1) return 0;
  const int nch = (vocab + kChunk - 1) / kChunk;
  return node_ws_layout(batch, (int64_t)batch * n_max, nch, nullptr, nullptr);
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
    hipLaunchKernelGGL(greedy_walk_kernel, dim3((unsigned)batch), dim3(64), 0, st, a);
    SPEC_LAUNCH_CHECK();
    return SPEC_OK;
  }
  const int64_t nodes = (int64_t)batch * n_max;
  if (!workspace || workspace_bytes < node_ws_layout(batch, nodes, nch, nullptr, nullptr)) return SPEC_ERR_WORKSPACE;
  if (nodes > 0x7fffffffLL || nodes * nch > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  const bool chunked = nch >= 2;
  NodeWs w{};
  node_ws_layout(batch, nodes, nch, (char*)workspace, &w);
  hipLaunchKernelGGL(plan_kernel, dim3((unsigned)nodes), dim3(192), 0, st, a, w, chunked ? 1 : 0);
  SPEC_LAUNCH_CHECK();
  if (chunked) {
    // grid-stride over (active node, chunk) items; the item count is known on the device only
    const int64_t upper = nodes * nch;
    const int64_t grid = std::min<int64_t>(upper, std::max<int64_t>(256, upper / 4));
    hipLaunchKernelGGL(chain_hist_kernel, dim3((unsigned)grid), dim3(kCThreads), 0, st, a, w);
    SPEC_LAUNCH_CHECK();
    hipLaunchKernelGGL(chain_exact_kernel, dim3((unsigned)grid), dim3(kXThreads), 0, st, a, w);
    SPEC_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(node_kernel, dim3((unsigned)nodes), dim3(kRjThreads), 0, st, a, w, chunked ? 1 : 0);
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}
