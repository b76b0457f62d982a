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
// the root then only follows the per-node results.  Large vocabularies (two or
// more chunks) add two launches before that, so that no workgroup ever waits for
// another:
//   R1  every internal node whose first child is rejected, one workgroup per
//       4096-token chunk: histogram of rho over 128 buckets per octave on [1, 16)
//       (two more just below 1, one for rho >= 16 or q == 0).  The bucket comes
//       from an fp32 log-domain estimate whose error is far below the 1% of a
//       bucket assumed everywhere; the bucket sums of p and q are exact.
//   R2  the same nodes and chunks: from the merged histogram, rigorous intervals
//       I_l holding c_{l+1} for every level l; then exact sums of p and q over
//       tokens with rho above each interval, the few tokens inside an interval in
//       a per-node list, and per-chunk sums for the terminal draw.  Only tokens in
//       buckets that straddle an interval end get an exact fp64 ratio.
//   R3  one workgroup per node: sibling tests with exact W(c_j) from R2's sums and
//       list, terminal draws located by exact chunk sums and one chunk scan; the
//       last workgroup of a request walks from the root and writes the outputs.
// All sums of p and q are kept in 2^-62 fixed point, so they are exact, independent
// of summation order and bitwise reproducible.  Small vocabularies (one chunk) and
// any case outside the fast path's guarantees (list or queue overflow, threshold
// beyond the histogram range, zero-mass steps) take direct vocabulary passes in R3.
#include "common.hpp"

namespace spectree {

constexpr int kHB = 512;            // ratio buckets over [1, 16): 128 per octave
constexpr int kHLow = 2;            // buckets just below rho = 1
constexpr int kHTop = kHB + kHLow;  // rho >= 16 or q == 0
constexpr int kHN = kHTop + 1;
constexpr double kHMargin = 0.01;   // bound on the estimate's error, in buckets
constexpr int kMaxKids = 63;        // chain levels per node
constexpr int kListCap = 4096;      // exact in-interval tokens kept per node
constexpr int kWgList = 256;        // in-interval tokens one R2 workgroup can stage
constexpr int kQueue = 1024;        // edge tokens one R2 workgroup can stage
constexpr int kLdsList = 512;       // list entries R3 keeps in LDS
constexpr int kMaxEdge = 24;        // edge buckets per level before the direct path
constexpr double kFx = 4611686018427387904.0;  // 2^62
constexpr double kFxInv = 1.0 / kFx;
constexpr int kRjThreads = 256;
constexpr int kFlagFallback = 1;

struct ListEntry {
  double p, q, rho;
  int32_t tok, pad;
};
struct QEntry {
  int32_t tok, h;
  float pp, qq;  // unnormalised fp32 masses
};
struct NodeRes {
  int32_t acc, term, err, pad;
};

struct NodeWs {         // per-node slots, nd = b * n_max + n
  NodeRes* res;         // [nd]                     R3 -> its request's last workgroup
  uint32_t* req_count;  // [batch]                  self-resetting
  long long* hist;      // [nd][kHN][2]             R1 -> R2 (cleared by R2)
  long long* lvl;       // [nd][kMaxKids][2]        R2 -> R3 (cleared by R1)
  double* ivl;          // [nd][kMaxKids][2]        R2 -> R3
  long long* cdraw;     // [nd][nch][2]             R2 -> R3
  ListEntry* list;      // [nd][kListCap]           R2 -> R3
  uint32_t* list_n;     // [nd]                     (cleared by R1)
  uint32_t* r2_count;   // [nd]                     self-resetting
  int32_t* flags;       // [nd]                     (cleared by R1)
};

struct RejArgs {
  const float *tgt_logits, *tgt_max, *tgt_sumexp;
  const int32_t* tgt_argmax;
  const float* tgt_chunk_max;
  const double* tgt_chunk_sum;
  const float *dft_logits, *dft_max, *dft_sumexp;
  double inv_t, inv_td;
  ExpScale est, esd;
  int greedy;
  const int32_t *tokens, *parent, *n_nodes;
  const float *u_accept, *u_sample;
  int32_t batch, n_max, vocab, nch;
  int32_t vec;  // rows start 16-byte aligned (vocab % 4 == 0, aligned bases)
  int32_t *accepted_child, *term_token, *status;
};

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

__device__ inline long long to_fx(double v) { return __double2ll_rz(v * kFx); }

struct RowView {
  const float* lt;
  const float* ld;
  float mt, md;
  double izt, izd;
};

// Row view of node row `row`; false if either row's statistics are invalid.
__device__ inline bool row_view(const RejArgs& a, int64_t row, RowView& r) {
  r.lt = a.tgt_logits + row * (int64_t)a.vocab;
  r.ld = a.dft_logits + row * (int64_t)a.vocab;
  r.mt = a.tgt_max[row];
  r.md = a.dft_max[row];
  if (isnan(r.mt) || isnan(r.md)) return false;
  r.izt = 1.0 / (double)a.tgt_sumexp[row];
  r.izd = 1.0 / (double)a.dft_sumexp[row];
  return true;
}
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
// Tested tokens: fp64 exp.
__device__ inline double p_tok(const RejArgs& a, const RowView& r, int x) {
  return exp(((double)r.lt[x] - (double)r.mt) * a.inv_t) * r.izt;
}
__device__ inline double q_tok(const RejArgs& a, const RowView& r, int x) {
  return exp(((double)r.ld[x] - (double)r.md) * a.inv_td) * r.izd;
}
// Acceptance ratio r(x)/q(x) with r = max(0, p - c q) / W.
__device__ inline double accept_ratio(double px, double qx, double c, double W) {
  const double num = fmax(0.0, px - c * qx);
  if (qx > 0.0) return num / (W * qx);
  return num > 0.0 ? INFINITY : 0.0;
}

// Node n of a request with nb nodes: number of children, first child (-1 if none).
__device__ inline int count_kids(const int* s_par, int n, int nb, int& first) {
  int k = 0;
  first = -1;
  for (int c = n + 1; c < nb; ++c)
    if (s_par[c] == n) {
      if (first < 0) first = c;
      ++k;
    }
  return k;
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
  if (!(pp > 0.0f)) return -1;
  if (!(qq > 0.0f)) return kHTop;
  const float x = floorf(__fmul_rn(__fadd_rn(__fsub_rn(ep, eq), K), 128.0f));
  if (x >= (float)kHB) return kHTop;
  if (x < (float)-kHLow) return -1;
  return (int)x + kHLow;
}
__device__ inline float row_k(const RejArgs& a, int64_t row) {
  return (float)(log2((double)a.dft_sumexp[row]) - log2((double)a.tgt_sumexp[row]));
}
// Certain ratio range of each bucket: lb[h] <= rho < ub[h].
__device__ inline void fill_edges(double* lb, double* ub) {
  for (int h = threadIdx.x; h < kHN; h += blockDim.x) {
    const double beta = (double)(h - kHLow);
    if (h == kHTop) {
      lb[h] = exp2(((double)kHB - kHMargin) / 128.0);
      ub[h] = INFINITY;
    } else {
      lb[h] = exp2((beta - kHMargin) / 128.0);
      ub[h] = exp2((beta + 1.0 + kHMargin) / 128.0);
    }
  }
}
__device__ inline int bucket_guess(double c) {
  const int i = (int)floorf(log2f((float)c) * 128.0f) + kHLow;
  return min(max(i, 0), kHTop);
}
// First bucket all of whose tokens have rho > c (kHN if none).
__device__ inline int first_above(double c, const double* lb) {
  int i = bucket_guess(c);
  while (i > 0 && lb[i - 1] > c) --i;
  while (i <= kHTop && !(lb[i] > c)) ++i;
  return i;
}
// First bucket that may hold a token with rho > c.
__device__ inline int first_maybe(double c, const double* ub) {
  int i = bucket_guess(c);
  while (i > 0 && ub[i - 1] > c) --i;
  while (i <= kHTop && !(ub[i] > c)) ++i;
  return i;
}

// Shared prelude of R1 and R2.  A workgroup serves one chunk of one node.
struct NodeJob {
  int b, n, nd, chunk, nb, k, first;
  int64_t row;
  RowView rv;
  float K;
};
// The tree of the node's request into LDS; false if the node has no children.
__device__ bool node_tree(const RejArgs& a, int* s_par, int* s_tok, NodeJob& j) {
  j.nd = blockIdx.x / a.nch;
  j.chunk = blockIdx.x % a.nch;
  j.b = j.nd / a.n_max;
  j.n = j.nd % a.n_max;
  j.row = j.nd;
  const int64_t base = (int64_t)j.b * a.n_max;
  if (threadIdx.x < 64) {
    const bool in = (int)threadIdx.x < a.n_max;
    s_par[threadIdx.x] = in ? a.parent[base + threadIdx.x] : -2;
    s_tok[threadIdx.x] = in ? a.tokens[base + threadIdx.x] : 0;
  }
  j.nb = a.n_nodes[j.b];
  __syncthreads();
  if (j.nb < 1 || j.nb > a.n_max || j.n >= j.nb) return false;
  j.k = count_kids(s_par, j.n, j.nb, j.first);
  return j.k > 0;
}
// Whether the node's first child is rejected: only then is its chain needed.  The
// test is the one R3 makes (residual p, c = 0, W = 1).
__device__ bool first_rejected(const RejArgs& a, const int* s_tok, NodeJob& j) {
  const int x = __builtin_amdgcn_readfirstlane(s_tok[j.first]);
  if (x < 0 || x >= a.vocab) return false;
  if (!row_view(a, j.row, j.rv)) return false;
  j.K = row_k(a, j.row);
  const double ratio = accept_ratio(p_tok(a, j.rv, x), q_tok(a, j.rv, x), 0.0, 1.0);
  return !((double)a.u_accept[(int64_t)j.b * a.n_max + j.first] < ratio);
}

__device__ inline long long wave_sum_ll(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
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

// ---------------------------------------------------------------------------
// R1: ratio histogram
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chain_hist_kernel(RejArgs a, NodeWs w) {
  __shared__ int s_par[64], s_tok[64];
  __shared__ unsigned long long s_P[4][kHN], s_Q[4][kHN];  // one copy per wavefront
  NodeJob j;
  if (!node_tree(a, s_par, s_tok, j)) return;
  const int tid = threadIdx.x, wv = tid >> 6;
  float xl[kPer], xd[kPer];  // issued before the first-child test, which needs other rows
  load_chunk(a.tgt_logits + j.row * a.vocab, j.chunk * kChunk, a.vocab, a.vec, xl);
  load_chunk(a.dft_logits + j.row * a.vocab, j.chunk * kChunk, a.vocab, a.vec, xd);
  if (!first_rejected(a, s_tok, j)) return;
  if (j.chunk == 0) {  // R2's accumulators for this node start from zero
    for (int i = tid; i < 2 * kMaxKids; i += blockDim.x) w.lvl[(int64_t)j.nd * 2 * kMaxKids + i] = 0;
    if (tid == 0) {
      w.list_n[j.nd] = 0;
      w.flags[j.nd] = 0;
    }
  }
  for (int i = tid; i < kHN; i += blockDim.x)
    for (int c = 0; c < 4; ++c) s_P[c][i] = s_Q[c][i] = 0;
  __syncthreads();
#pragma unroll
  for (int s2 = 0; s2 < kPer; ++s2) {
    const float ep = exp2_arg(xl[s2], j.rv.mt, a.est), eq = exp2_arg(xd[s2], j.rv.md, a.esd);
    const float pp = __builtin_amdgcn_exp2f(ep), qq = __builtin_amdgcn_exp2f(eq);
    const int h = est_bucket(ep, eq, pp, qq, j.K);
    if (h < 0) continue;
    atomicAdd(&s_P[wv][h], (unsigned long long)to_fx((double)pp * j.rv.izt));
    atomicAdd(&s_Q[wv][h], (unsigned long long)to_fx((double)qq * j.rv.izd));
  }
  __syncthreads();
  unsigned long long* hg = (unsigned long long*)w.hist + (int64_t)j.nd * 2 * kHN;
  for (int i = tid; i < kHN; i += blockDim.x) {
    const unsigned long long P = s_P[0][i] + s_P[1][i] + s_P[2][i] + s_P[3][i];
    const unsigned long long Q = s_Q[0][i] + s_Q[1][i] + s_Q[2][i] + s_Q[3][i];
    if (P) atomicAdd(&hg[2 * i], P);
    if (Q) atomicAdd(&hg[2 * i + 1], Q);
  }
}

// ---------------------------------------------------------------------------
// R2: chain intervals and exact sums
// ---------------------------------------------------------------------------
// Bounds of W(c) from the histogram's suffix sums S (fixed point, scaled back):
// buckets from first_above(c) count in full; the one or two buckets straddling c
// contribute between max(0, P - cQ) (jointly) and (ub - c) Q each.
__device__ void w_bounds(double c, const double* lb, const double* ub, const long long* S, double& lo,
                         double& hi) {
  const int ia = first_above(c, lb), im = first_maybe(c, ub);
  const double full = ia < kHN ? ((double)S[2 * ia] - c * (double)S[2 * ia + 1]) * kFxInv : 0.0;
  double up = 0.0, uq = 0.0, extra = 0.0;
  for (int i = im; i < ia && i < kHN; ++i) {
    const double P = (double)(S[2 * i] - S[2 * i + 2]) * kFxInv, Q = (double)(S[2 * i + 1] - S[2 * i + 3]) * kFxInv;
    up += P;
    uq += Q;
    if (Q > 0.0) extra += isinf(ub[i]) ? INFINITY : fmax(0.0, (ub[i] - c) * Q);
    else extra += P;  // q == 0 tokens count in full
  }
  lo = full + fmax(0.0, up - c * uq);
  hi = full + extra;
}

// Pushes v onto the LDS queue for the lanes with e set (one LDS atomic per wave).
__device__ inline void queue_push(bool e, const QEntry& v, QEntry* q, int* qn) {
  const unsigned long long m = __ballot(e);
  if (m == 0) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)m) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(qn, __popcll(m));
  base = __shfl(base, leader);
  const int off = __popcll(m & ((1ull << lane) - 1ull));
  if (e && base + off < kQueue) q[base + off] = v;
}

// Levels: l = 0 .. k-1 is the threshold after l + 1 rejections, c_{l+1} in
// I_l = [a_l, b_l] (I_0 = [1, 1]).  With H_l the first bucket certainly above b_l
// and G_l the first bucket that may hold rho > a_l:
//   P_above(l) = sum_{rho > b_l} p = S[H_l] + (tokens of buckets [G_l, H_l) with rho > b_l),
// and the tokens of [G_l, H_l) with a_l < rho <= b_l are kept in the node's list.
__global__ __launch_bounds__(256) void chain_exact_kernel(RejArgs a, NodeWs w) {
  __shared__ int s_par[64], s_tok[64];
  __shared__ double s_lb[kHN], s_ub[kHN];
  __shared__ long long s_S[2 * (kHN + 1)];  // suffix sums of the merged histogram
  __shared__ long long s_wt[2][4];
  __shared__ double s_a[kMaxKids], s_b[kMaxKids];
  __shared__ int s_G[kMaxKids], s_H[kMaxKids];
  __shared__ unsigned char s_edge[kHN];
  __shared__ unsigned long long s_EP[kMaxKids], s_EQ[kMaxKids];
  __shared__ QEntry s_q[kQueue];
  __shared__ ListEntry s_list[kWgList];
  __shared__ long long s_ll[4];
  __shared__ int s_qn, s_nlist, s_base, s_clear, s_bad, s_htop;
  NodeJob j;
  if (!node_tree(a, s_par, s_tok, j)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  float xl[kPer], xd[kPer];
  load_chunk(a.tgt_logits + j.row * a.vocab, j.chunk * kChunk, a.vocab, a.vec, xl);
  load_chunk(a.dft_logits + j.row * a.vocab, j.chunk * kChunk, a.vocab, a.vec, xd);
  if (!first_rejected(a, s_tok, j)) return;
  const long long* hg = w.hist + (int64_t)j.nd * 2 * kHN;
  // suffix sums S[h] = sum_{h' >= h} hist[h'] (S[kHN] = 0): thread t owns buckets 3t .. 3t+2
  long long v0[3], v1[3];
#pragma unroll
  for (int e = 0; e < 3; ++e) {
    const int h = 3 * tid + e;
    v0[e] = h < kHN ? hg[2 * h] : 0;
    v1[e] = h < kHN ? hg[2 * h + 1] : 0;
  }
  fill_edges(s_lb, s_ub);
  for (int i = tid; i < kHN; i += blockDim.x) s_edge[i] = 0;
  for (int i = tid; i < kMaxKids; i += blockDim.x) s_EP[i] = s_EQ[i] = 0;
  if (tid == 0) {
    s_qn = 0;
    s_nlist = 0;
  }
  {
    const long long t0 = v0[0] + v0[1] + v0[2], t1 = v1[0] + v1[1] + v1[2];
    long long i0 = t0, i1 = t1;  // inclusive suffix within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long u0 = __shfl_down(i0, o), u1 = __shfl_down(i1, o);
      if (lane + o < 64) {
        i0 += u0;
        i1 += u1;
      }
    }
    if (lane == 0) {
      s_wt[0][wv] = i0;
      s_wt[1][wv] = i1;
    }
    __syncthreads();
    long long e0 = i0 - t0, e1 = i1 - t1;  // exclusive suffix
    for (int x = wv + 1; x < 4; ++x) {
      e0 += s_wt[0][x];
      e1 += s_wt[1][x];
    }
    for (int e = 2; e >= 0; --e) {
      e0 += v0[e];
      e1 += v1[e];
      const int h = 3 * tid + e;
      if (h <= kHN) {
        s_S[2 * h] = e0;
        s_S[2 * h + 1] = e1;
      }
    }
  }
  __syncthreads();
  // every workgroup of this node has read the histogram: the last one clears it
  if (tid == 0) s_clear = pub_arrive(&w.r2_count[j.nd]) == (uint32_t)(a.nch - 1);
  __syncthreads();
  if (s_clear) {
    long long* hw = w.hist + (int64_t)j.nd * 2 * kHN;
    for (int i = tid; i < 2 * kHN; i += blockDim.x) hw[i] = 0;
    if (tid == 0) w.r2_count[j.nd] = 0;
  }
  const int k = j.k;
  if (tid == 0) {  // intervals and their bucket ranges
    int bad = 0;
    s_a[0] = s_b[0] = 1.0;
    for (int l = 1; l < k; ++l) {
      double lo1, hi1, lo2, hi2;
      w_bounds(s_a[l - 1], s_lb, s_ub, s_S, lo1, hi1);
      w_bounds(s_b[l - 1], s_lb, s_ub, s_S, lo2, hi2);
      const double na = s_a[l - 1] + lo1, nb = s_b[l - 1] + hi2;
      const double pad = 1e-7 * (nb - na) + 1e-12 * nb;
      s_a[l] = na - pad;
      s_b[l] = nb + pad;
      if (!(s_b[l] < 16.0)) {
        bad = 1;
        break;
      }
    }
    for (int l = 0; l < k && !bad; ++l) {
      s_G[l] = first_maybe(s_a[l], s_ub);
      s_H[l] = first_above(s_b[l], s_lb);
      if (s_H[l] > kHTop || s_H[l] - s_G[l] > kMaxEdge) bad = 1;  // outside the histogram: direct path
    }
    if (!bad) {
      for (int l = 0; l < k; ++l)
        for (int i = s_G[l]; i < s_H[l]; ++i) s_edge[i] = 1;
      s_htop = s_H[k - 1];
    }
    s_bad = bad;
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) atomicOr(&w.flags[j.nd], kFlagFallback);
    return;
  }
  if (j.chunk == 0) {  // the certain parts above each interval, and the intervals
    unsigned long long* lv = (unsigned long long*)w.lvl + (int64_t)j.nd * 2 * kMaxKids;
    for (int l = tid; l < k; l += blockDim.x) {
      const int i = s_H[l];
      if (s_S[2 * i]) atomicAdd(&lv[2 * l], (unsigned long long)s_S[2 * i]);
      if (s_S[2 * i + 1]) atomicAdd(&lv[2 * l + 1], (unsigned long long)s_S[2 * i + 1]);
      w.ivl[((int64_t)j.nd * kMaxKids + l) * 2] = s_a[l];
      w.ivl[((int64_t)j.nd * kMaxKids + l) * 2 + 1] = s_b[l];
    }
  }
  const int htop = s_htop;
  const double btop = s_b[k - 1];
  long long cp = 0, cq = 0;  // this chunk's tokens with rho > b_{k-1} (the terminal draw)
#pragma unroll
  for (int s2 = 0; s2 < kPer; ++s2) {
    const float ep = exp2_arg(xl[s2], j.rv.mt, a.est), eq = exp2_arg(xd[s2], j.rv.md, a.esd);
    const float pp = __builtin_amdgcn_exp2f(ep), qq = __builtin_amdgcn_exp2f(eq);
    const int h = est_bucket(ep, eq, pp, qq, j.K);
    if (h >= htop) {
      cp += to_fx((double)pp * j.rv.izt);
      cq += to_fx((double)qq * j.rv.izd);
    }
    const bool edge = h >= 0 && h < htop && s_edge[h];
    queue_push(edge, QEntry{chunk_tok(j.chunk * kChunk, s2), h, pp, qq}, s_q, &s_qn);
  }
  __syncthreads();
  const int qn = s_qn;
  for (int i = tid; i < min(qn, kQueue); i += blockDim.x) {
    const QEntry e = s_q[i];
    const double p = (double)e.pp * j.rv.izt, q = (double)e.qq * j.rv.izd;
    const double rho = q > 0.0 ? p / q : INFINITY;
    const long long fp = to_fx(p), fq = to_fx(q);
    if (rho > btop) {
      cp += fp;
      cq += fq;
    }
    bool in_list = false;
    for (int l = 0; l < k; ++l) {
      if (e.h < s_G[l] || e.h >= s_H[l]) continue;
      if (rho > s_b[l]) {
        if (fp) atomicAdd(&s_EP[l], (unsigned long long)fp);
        if (fq) atomicAdd(&s_EQ[l], (unsigned long long)fq);
      } else if (rho > s_a[l]) {
        in_list = true;
      }
    }
    if (in_list) {
      const int x = atomicAdd(&s_nlist, 1);
      if (x < kWgList) s_list[x] = ListEntry{p, q, rho, e.tok, 0};
    }
  }
  cp = block_sum_ll(cp, s_ll);
  cq = block_sum_ll(cq, s_ll);
  if (tid == 0) {
    long long* cd = w.cdraw + ((int64_t)j.nd * a.nch + j.chunk) * 2;
    cd[0] = cp;
    cd[1] = cq;
    const int n_in = s_nlist;
    if (qn > kQueue || n_in > kWgList) {
      atomicOr(&w.flags[j.nd], kFlagFallback);
      s_base = -1;
    } else {
      s_base = n_in ? (int)atomicAdd(&w.list_n[j.nd], (uint32_t)n_in) : 0;
      if (s_base + n_in > kListCap) atomicOr(&w.flags[j.nd], kFlagFallback);
    }
  }
  unsigned long long* lv = (unsigned long long*)w.lvl + (int64_t)j.nd * 2 * kMaxKids;
  for (int l = tid; l < k; l += blockDim.x) {
    if (s_EP[l]) atomicAdd(&lv[2 * l], s_EP[l]);
    if (s_EQ[l]) atomicAdd(&lv[2 * l + 1], s_EQ[l]);
  }
  __syncthreads();
  const int n_in = min(s_nlist, kWgList);
  if (s_base >= 0)
    for (int i = tid; i < n_in; i += blockDim.x)
      if (s_base + i < kListCap) w.list[(int64_t)j.nd * kListCap + s_base + i] = s_list[i];
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
__device__ int scan_range(int t0, int t1, double pre, double target, Elem elem, double* s_scan, int* s_pick) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (t1 - t0 + nt - 1) / nt;
  const int r0 = t0 + tid * per, r1 = min(t1, r0 + per);
  double own = 0.0;
  for (int t = r0; t < r1; ++t) own += elem(t);
  __syncthreads();
  s_scan[tid] = own;
  if (tid == 0) *s_pick = 0x7fffffff;
  __syncthreads();
  if (tid == 0) {  // exclusive prefix in thread order
    double run = 0.0;
    for (int i = 0; i < nt; ++i) {
      const double v = s_scan[i];
      s_scan[i] = run;
      run += v;
    }
  }
  __syncthreads();
  const double before = pre + s_scan[tid];
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
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o));
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
                          double c, double pre, double target, double* s_scan, int* s_pick) {
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
  __syncthreads();
  s_scan[tid] = own;
  if (tid == 0) *s_pick = 0x7fffffff;
  __syncthreads();
  if (tid == 0) {  // exclusive prefix in thread order
    double run = 0.0;
    for (int i = 0; i < (int)blockDim.x; ++i) {
      const double v = s_scan[i];
      s_scan[i] = run;
      run += v;
    }
  }
  __syncthreads();
  const double before = pre + s_scan[tid];
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
__device__ int direct_draw(const RejArgs& a, const RowView& r, double c, double u, double* s_red, double* s_scan,
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
      int k = scan_range(t0, t1, pre, target, el, s_scan, s_pick);
      if (k < 0) k = last_positive(0, a.vocab, el, s_pick);
      return k;
    }
    pre += sc;
  }
  return -1;
}

// Chunk holding the target u * sum(s_chunk) in the exact per-chunk masses s_chunk;
// *pre is the mass of the chunks before it.
__device__ inline int pick_chunk(const double* s_chunk, int nch, double u, double* pre, double* target) {
  double S = 0.0;
  for (int ch = 0; ch < nch; ++ch) S += s_chunk[ch];
  *target = u * S;
  double run = 0.0;
  int ch = 0;
  for (; ch < nch - 1; ++ch) {
    if (run + s_chunk[ch] > *target) break;
    run += s_chunk[ch];
  }
  *pre = run;
  return ch;
}

// One workgroup per node slot.  Node results go to the workspace; the request's
// last workgroup walks from the root and writes accepted_child / term_token.
__global__ __launch_bounds__(kRjThreads) void node_kernel(RejArgs a, NodeWs w, int chunked) {
  __shared__ int s_par[64], s_tok[64];
  __shared__ float s_ua[64], s_xl[64], s_xd[64];
  __shared__ long long s_lv[2 * kMaxKids];
  __shared__ double s_iv[2 * kMaxKids];
  __shared__ ListEntry s_list[kLdsList];
  __shared__ double s_red[kRjThreads / 64];
  __shared__ long long s_ll[kRjThreads / 64];
  __shared__ double s_scan[kRjThreads];
  __shared__ double s_chunk[256];
  __shared__ unsigned long long s_cP[256], s_cQ[256];
  __shared__ int s_pick, s_bad, s_flag, s_nlist, s_last;
  __shared__ NodeRes s_res[64];
  __shared__ int s_oacc[64], s_oterm[64];
  const int tid = threadIdx.x;
  const int nd = blockIdx.x;
  const int b = nd / a.n_max, n = nd % a.n_max;
  const int64_t base = (int64_t)b * a.n_max, row = nd;
  if (tid < 64) {
    const bool in = tid < a.n_max;
    s_par[tid] = in ? a.parent[base + tid] : -2;
    s_tok[tid] = in ? a.tokens[base + tid] : 0;
    s_ua[tid] = in ? a.u_accept[base + tid] : 0.0f;
  }
  if (tid == 0) s_bad = 0;
  const int nb = a.n_nodes[b];
  const bool n_ok = nb >= 1 && nb <= a.n_max;
  RowView rv;
  rv.lt = a.tgt_logits + row * (int64_t)a.vocab;
  rv.ld = a.dft_logits + row * (int64_t)a.vocab;
  rv.mt = a.tgt_max[row];
  rv.md = a.dft_max[row];
  const float zt = a.tgt_sumexp[row], zd = a.dft_sumexp[row];
  const float us = a.u_sample[row];
  __syncthreads();
  // the request's tree: parents precede children, tokens in range
  if (n_ok && tid < nb) {
    const int p = s_par[tid];
    if (tid == 0 ? p != -1 : (p < 0 || p >= tid)) atomicOr(&s_bad, 1);
    else if (tid > 0 && (s_tok[tid] < 0 || s_tok[tid] >= a.vocab)) atomicOr(&s_bad, 2);
  }
  __syncthreads();
  NodeRes res{SPEC_NODE_NOT_EVALUATED, SPEC_NODE_NOT_EVALUATED, 0, 0};
  if (n_ok && s_bad == 0 && n < nb) {
    if (isnan(rv.mt) || isnan(rv.md)) {
      res.err = 1;
    } else {
      rv.izt = 1.0 / (double)zt;
      rv.izd = 1.0 / (double)zd;
      int first;
      const int k = count_kids(s_par, n, nb, first);
      if (tid > n && tid < nb && s_par[tid] == n) {  // the children's tokens in this row
        s_xl[tid] = rv.lt[s_tok[tid]];
        s_xd[tid] = rv.ld[s_tok[tid]];
      }
      if (k > 0 && chunked) {
        for (int i = tid; i < 2 * k; i += blockDim.x) {
          s_lv[i] = w.lvl[(int64_t)nd * 2 * kMaxKids + i];
          s_iv[i] = w.ivl[(int64_t)nd * kMaxKids * 2 + i];
        }
        if (tid == 0) {
          s_flag = w.flags[nd];
          s_nlist = (int)min(w.list_n[nd], (uint32_t)kListCap);
        }
      }
      __syncthreads();
      int acc = SPEC_NODE_NONE, term = -1;
      if (k == 0) {
        // ---- leaf: the bonus is drawn from p ----
        const double u = (double)us;
        if (chunked && a.tgt_chunk_max) {
          const float* cmx = a.tgt_chunk_max + row * a.nch;
          const double* csm = a.tgt_chunk_sum + row * a.nch;
          if (tid < a.nch) s_chunk[tid] = csm[tid] * exp(((double)cmx[tid] - (double)rv.mt) * a.inv_t);
          __syncthreads();
          double pre, target;
          const int ch = pick_chunk(s_chunk, a.nch, u, &pre, &target);
          const float mc = cmx[ch];
          const double scale = exp(((double)mc - (double)rv.mt) * a.inv_t);
          const int t0 = ch * kChunk, t1 = min(a.vocab, t0 + kChunk);
          term = chunk_scan(a, rv, t0, t1, false, mc, scale, 0.0, pre, target, s_scan, &s_pick);
          if (term < 0) {
            auto el = [&](int t) { return (double)exp_scaled(rv.lt[t] - mc, a.est) * scale; };
            term = last_positive(t0, t1, el, &s_pick);
          }
        } else {
          term = direct_draw(a, rv, 0.0, u, s_red, s_scan, &s_pick);
        }
      } else {
        // ---- children in ascending index, tested against the running residual ----
        const bool fast = chunked && !(s_flag & kFlagFallback);
        const ListEntry* L = w.list + (int64_t)nd * kListCap;
        const int nlist = fast ? s_nlist : 0;
        const bool in_lds = nlist <= kLdsList;
        if (in_lds)
          for (int i = tid; i < nlist; i += blockDim.x) s_list[i] = L[i];
        const ListEntry* LL = in_lds ? s_list : L;
        __syncthreads();
        int lvl = 0;  // rejections so far
        double c = 0.0, W = 1.0;
        bool fell_back = !fast, zero_last = false;
        for (int ci = first; ci < nb; ++ci) {
          if (s_par[ci] != n) continue;
          const double px = exp(((double)s_xl[ci] - (double)rv.mt) * a.inv_t) * rv.izt;
          const double qx = exp(((double)s_xd[ci] - (double)rv.md) * a.inv_td) * rv.izd;
          if ((double)s_ua[ci] < accept_ratio(px, qx, c, W)) {
            acc = ci;
            break;
          }
          ++lvl;  // cn = c + W is the threshold after this rejection
          const double cn = c + W;
          double Wn = 0.0;
          if (!fell_back) {
            const double ia = s_iv[2 * (lvl - 1)], ib = s_iv[2 * (lvl - 1) + 1];
            if (!(cn >= ia && cn <= ib)) {
              fell_back = true;
            } else {
              long long lp = 0, lq = 0;  // listed tokens inside the interval and above cn
              for (int i = tid; i < nlist; i += blockDim.x) {
                const ListEntry e = LL[i];
                if (e.rho > cn && e.rho <= ib) {
                  lp += to_fx(e.p);
                  lq += to_fx(e.q);
                }
              }
              lp = block_sum_ll(lp, s_ll);
              lq = block_sum_ll(lq, s_ll);
              Wn = ((double)(s_lv[2 * (lvl - 1)] + lp) - cn * (double)(s_lv[2 * (lvl - 1) + 1] + lq)) * kFxInv;
            }
          }
          if (fell_back) Wn = direct_W(a, rv, cn, s_red);
          if (Wn > 0.0) {
            c = cn;
            W = Wn;
            zero_last = false;
          } else {
            zero_last = true;  // the residual keeps its previous threshold
          }
        }
        if (acc < 0) {
          // ---- all children rejected: the bonus is drawn from the residual ----
          const double u = (double)us;
          if (!fell_back && !zero_last) {
            const double ib = s_iv[2 * (k - 1) + 1];
            const long long* cd = w.cdraw + (int64_t)nd * a.nch * 2;
            for (int ch = tid; ch < a.nch; ch += blockDim.x) {
              s_cP[ch] = (unsigned long long)cd[2 * ch];
              s_cQ[ch] = (unsigned long long)cd[2 * ch + 1];
            }
            __syncthreads();
            for (int i = tid; i < nlist; i += blockDim.x) {
              const ListEntry e = LL[i];
              if (e.rho > c && e.rho <= ib) {
                const int ch = e.tok / kChunk;
                atomicAdd(&s_cP[ch], (unsigned long long)to_fx(e.p));
                atomicAdd(&s_cQ[ch], (unsigned long long)to_fx(e.q));
              }
            }
            __syncthreads();
            if (tid < a.nch)
              s_chunk[tid] = ((double)(long long)s_cP[tid] - c * (double)(long long)s_cQ[tid]) * kFxInv;
            __syncthreads();
            double pre, target;
            const int ch = pick_chunk(s_chunk, a.nch, u, &pre, &target);
            const int t0 = ch * kChunk, t1 = min(a.vocab, t0 + kChunk);
            term = chunk_scan(a, rv, t0, t1, true, 0.0f, 1.0, c, pre, target, s_scan, &s_pick);
            if (term < 0) {
              const double cc = c;
              auto el = [&](int t) { return resid_el(a, rv, t, cc); };
              term = last_positive(t0, t1, el, &s_pick);
            }
          } else {
            term = direct_draw(a, rv, c, u, s_red, s_scan, &s_pick);
          }
        }
      }
      res.acc = acc;
      res.term = acc >= 0 ? SPEC_NODE_NOT_EVALUATED : term;
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
  }
  if (tid < 64) {
    s_oacc[tid] = SPEC_NODE_NOT_EVALUATED;
    s_oterm[tid] = SPEC_NODE_NOT_EVALUATED;
  }
  __syncthreads();
  if (tid == 0) {
    pub_store(&w.req_count[b], 0u);
    int verdict = !n_ok || (s_bad & 1) ? SPEC_ERR_BAD_TREE : (s_bad ? SPEC_ERR_BAD_INPUT : 0);
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
}

// T == 0: one wavefront per request follows the target argmax.
__global__ __launch_bounds__(64) void greedy_walk_kernel(RejArgs a) {
  __shared__ int s_par[64], s_tok[64], s_arg[64], s_oacc[64], s_oterm[64];
  __shared__ float s_max[64];
  __shared__ int s_bad;
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
}

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout: node results and request counters always; the chain arrays
// when the vocabulary spans two or more chunks.
inline size_t node_ws_layout(int64_t batch, int64_t nodes, int nch, char* base, NodeWs* w) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += a256(bytes);
    return p;
  };
  NodeWs t{};
  t.res = (NodeRes*)take((size_t)nodes * sizeof(NodeRes));
  t.req_count = (uint32_t*)take((size_t)batch * 4);
  if (nch >= 2) {
    t.hist = (long long*)take((size_t)nodes * kHN * 16);
    t.lvl = (long long*)take((size_t)nodes * kMaxKids * 16);
    t.ivl = (double*)take((size_t)nodes * kMaxKids * 16);
    t.cdraw = (long long*)take((size_t)nodes * nch * 16);
    t.list = (ListEntry*)take((size_t)nodes * kListCap * sizeof(ListEntry));
    t.list_n = (uint32_t*)take((size_t)nodes * 4);
    t.r2_count = (uint32_t*)take((size_t)nodes * 4);
    t.flags = (int32_t*)take((size_t)nodes * 4);
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

extern "C" int spec_tree_reject_sample(const float* tgt_logits, const float* tgt_max, const float* tgt_sumexp,
                                       const int32_t* tgt_argmax, const float* tgt_chunk_max,
                                       const double* tgt_chunk_sum, float temperature, const float* dft_logits,
                                       const float* dft_max, const float* dft_sumexp, float draft_temperature,
                                       const int32_t* tokens, const int32_t* parent, const int32_t* n_nodes,
                                       const float* u_accept, const float* u_sample, int32_t batch, int32_t n_max,
                                       int32_t vocab, int32_t* accepted_child, int32_t* term_token, void* workspace,
                                       size_t workspace_bytes, int32_t* status, void* stream) {
  using namespace spectree;
  if (!(temperature >= 0.0f) || isinf(temperature)) return SPEC_ERR_INVALID_ARG;
  const bool greedy = temperature == 0.0f;
  if (!tgt_logits || !tgt_max || !tokens || !parent || !n_nodes || !accepted_child || !term_token)
    return SPEC_ERR_INVALID_ARG;
  if (greedy && !tgt_argmax) return SPEC_ERR_INVALID_ARG;
  if (!greedy) {
    if (!tgt_sumexp || !dft_logits || !dft_max || !dft_sumexp || !u_accept || !u_sample) return SPEC_ERR_INVALID_ARG;
    if (!(draft_temperature > 0.0f) || isinf(draft_temperature)) return SPEC_ERR_INVALID_ARG;
    if ((tgt_chunk_max == nullptr) != (tgt_chunk_sum == nullptr)) return SPEC_ERR_INVALID_ARG;
  }
  if (batch < 1 || n_max < 1 || n_max > 64 || vocab < 1) return SPEC_ERR_INVALID_ARG;
  const int nch = (vocab + kChunk - 1) / kChunk;
  if (nch > 256) return SPEC_ERR_UNSUPPORTED;
  const bool chunked = !greedy && nch >= 2;
  RejArgs a{};
  a.tgt_logits = tgt_logits;
  a.tgt_max = tgt_max;
  a.tgt_sumexp = tgt_sumexp;
  a.tgt_argmax = tgt_argmax;
  a.tgt_chunk_max = tgt_chunk_max;
  a.tgt_chunk_sum = tgt_chunk_sum;
  a.dft_logits = dft_logits;
  a.dft_max = dft_max;
  a.dft_sumexp = dft_sumexp;
  a.greedy = greedy ? 1 : 0;
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
  a.status = status;
  hipStream_t st = (hipStream_t)stream;
  if (greedy) {
    hipLaunchKernelGGL(greedy_walk_kernel, dim3((unsigned)batch), dim3(64), 0, st, a);
    SPEC_LAUNCH_CHECK();
    return SPEC_OK;
  }
  const int64_t nodes = (int64_t)batch * n_max;
  if (!workspace || workspace_bytes < node_ws_layout(batch, nodes, nch, nullptr, nullptr)) return SPEC_ERR_WORKSPACE;
  NodeWs w{};
  node_ws_layout(batch, nodes, nch, (char*)workspace, &w);
  if (nodes > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  if (chunked) {
    const int64_t grid = nodes * nch;
    if (grid > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(chain_hist_kernel, dim3((unsigned)grid), dim3(256), 0, st, a, w);
    SPEC_LAUNCH_CHECK();
    hipLaunchKernelGGL(chain_exact_kernel, dim3((unsigned)grid), dim3(256), 0, st, a, w);
    SPEC_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(node_kernel, dim3((unsigned)nodes), dim3(kRjThreads), 0, st, a, w, chunked ? 1 : 0);
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}
