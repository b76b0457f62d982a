// Draft-tree construction on the GPU: EAGLE-2 expand and rerank.
//
// Tree-verification notes (zhangshuibai.github.io), "Tree Verification 详解" part
// E.2: a node's value is the product of the draft confidences on its root path;
// each expand round takes the frontier nodes of largest value, and each of them gets
// the top-k tokens of its draft distribution as children; the rerank keeps the N
// nodes of largest value, which form a connected subtree because value never grows
// along a path.  "The EAGLE Family" (consciousengines.com), "EAGLE-2: context-aware
// dynamic trees": the kept nodes are flattened with a tree mask for verification.
//
// Per request the tree under construction lives in caller arrays indexed by node id
// (parent, token, path key, value in fp64, confidence).  One expand call is one
// round: the caller has run the drafter on the current frontier and passes one
// logit row per frontier node.
//   tb_topk_kernel    one workgroup per (request, frontier row, 4096-token chunk):
//                     one read of the chunk gives its maximum, its fp64 sum of
//                     exp((l - m_c) / T_d) and its top-k (logit, token) keys; the
//                     row's last workgroup to finish (agent-scope counter) merges the
//                     row's chunks and writes its children (value = parent value x
//                     confidence), so the rows merge on different CUs
//   tb_select_kernel  one workgroup per request: appends the children and picks
//                     the next frontier
// The rerank is one workgroup per request: a bitonic sort of every candidate by
// (value desc, depth asc, id asc) in LDS, the top N - 1 plus the root, then the
// breadth-first order from each node's path key (depth, then the sibling ranks of
// its ancestors from the root down), which orders by depth, parent position and
// sibling order at once.
#include "common.hpp"

namespace spectree {

constexpr int kTbThreads = 256;
constexpr int kTbPer = kChunk / kTbThreads;  // 16 logits per thread
constexpr int kTbMaxK = 16;                  // children per expanded node
constexpr int kTbMaxFrontier = 16;           // nodes expanded per round
constexpr int kTbMaxChunks = 64;             // vocabulary up to 64 chunks
constexpr int kTbMaxCap = 1024;              // candidates per request (sorted in LDS)
constexpr int kTbMaxDepth = 15;              // path keys hold 15 four-bit sibling ranks
constexpr int kTbRerankThreads = kTbMaxCap;  // one candidate per thread
constexpr int kTbCand = 128;                            // threshold candidates ranked directly
static_assert(kTbMaxFrontier * kTbMaxK <= kTbThreads, "one thread per new child");
typedef float tb_f32x4 __attribute__((ext_vector_type(4)));

inline size_t tb_align(size_t x) { return (x + 255) & ~(size_t)255; }

// Orderable key of (logit, token): a larger logit gives a larger key, and equal
// logits give the lower token the larger key.  Key 0 is no token.
__device__ inline uint64_t tb_key(float x, int t) {
  uint32_t u = __float_as_uint(x);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)t);
}
__device__ inline float tb_key_logit(uint64_t k) {
  uint32_t u = (uint32_t)(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(u);
}
__device__ inline int tb_key_token(uint64_t k) { return (int)(~(uint32_t)k); }

template <int kCtrl, int kRowMask = 0xf>
__device__ inline uint64_t max_dpp_u64(uint64_t v) {
  const uint64_t o = (uint64_t)dpp_ll<kCtrl, kRowMask>((long long)v, (long long)v);
  return o > v ? o : v;
}
__device__ inline uint64_t wave_max_u64(uint64_t v) {
  v = max_dpp_u64<kDppQuad1032>(v);
  v = max_dpp_u64<kDppQuad2301>(v);
  v = max_dpp_u64<kDppHalfMirror>(v);
  v = max_dpp_u64<kDppMirror>(v);
  v = max_dpp_u64<kDppBcast15, 0xa>(v);
  v = max_dpp_u64<kDppBcast31, 0xc>(v);
  return (uint64_t)lane63_ll((long long)v);
}

template <int kCtrl, int kRowMask = 0xf>
__device__ inline uint32_t max_dpp_u32(uint32_t v) {
  const uint32_t o = (uint32_t)dpp_i<kCtrl, kRowMask>((int)v, (int)v);
  return o > v ? o : v;
}
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max_dpp_u32<kDppQuad1032>(v);
  v = max_dpp_u32<kDppQuad2301>(v);
  v = max_dpp_u32<kDppHalfMirror>(v);
  v = max_dpp_u32<kDppMirror>(v);
  v = max_dpp_u32<kDppBcast15, 0xa>(v);
  v = max_dpp_u32<kDppBcast31, 0xc>(v);
  return (uint32_t)lane63_i((int)v);
}
// The same maximum in two 32-bit steps: the high words, then the low words of the
// lanes that hold the largest high word.
__device__ inline uint64_t wave_max_u64_2step(uint64_t v) {
  const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}

// (value desc, then t asc): t is depth << 10 | id in the rerank, the id in the best-first frontier
__device__ inline bool rr_before(double va, uint32_t ta, double vb, uint32_t tb) {
  return va > vb || (va == vb && ta < tb);
}

// (value desc, id asc) ordering of candidates and its wave-wide maximum.
__device__ inline bool tb_better(double v, int i, double ov, int oi) { return ov > v || (ov == v && oi < i); }
template <int kCtrl, int kRowMask = 0xf>
__device__ inline void best_dpp_vd(double& v, int& i) {
  const double ov = dpp_d<kCtrl, kRowMask>(v, v);
  const int oi = dpp_i<kCtrl, kRowMask>(i, i);
  if (tb_better(v, i, ov, oi)) {
    v = ov;
    i = oi;
  }
}
__device__ inline void wave_best_vd(double& v, int& i) {
  best_dpp_vd<kDppQuad1032>(v, i);
  best_dpp_vd<kDppQuad2301>(v, i);
  best_dpp_vd<kDppHalfMirror>(v, i);
  best_dpp_vd<kDppMirror>(v, i);
  best_dpp_vd<kDppBcast15, 0xa>(v, i);
  best_dpp_vd<kDppBcast31, 0xc>(v, i);
  v = lane63_d(v);
  i = lane63_i(i);
}

// This wavefront's LDS writes are visible to its own later LDS reads.
__device__ inline void wave_lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

struct TbArgs {
  const float* logits;  // [batch, R, vocab]
  int32_t vocab, nch, R, K, select_k, cap;
  int32_t policy;  // 0: next frontier among this round's children; 1: among every leaf
  double inv_t;
  ExpScale es;
  int32_t* parent;  // [batch, cap] ...
  int32_t* token;
  uint64_t* path;
  double* value;
  double* conf;
  int32_t* count;     // [batch]
  int32_t* frontier;  // [batch, R]
  int32_t* fcount;    // [batch]
  uint64_t* ws_keys;  // [batch, R, nch, kTbMaxK]  chunk partials
  float* ws_max;      // [batch, R, nch]
  double* ws_sum;
  int32_t* ws_bad;
  uint32_t* row_cnt;  // [batch, R]  chunk workgroups of the row done (0 between calls)
  double* row_val;    // [batch, R, kTbMaxK]  the row's children: value, confidence, token
  double* row_conf;
  int32_t* row_tok;
  int32_t* row_node;  // [batch, R]  the expanded node, its path key, an error flag
  uint64_t* row_path;
  int32_t* row_bad;
  int32_t* status;
};

inline size_t tb_ws_bytes(int64_t batch, int32_t R, int32_t nch) {
  const size_t n = (size_t)batch * (size_t)R * (size_t)nch, rows = (size_t)batch * (size_t)R;
  return tb_align(n * kTbMaxK * 8) + tb_align(n * 4) + tb_align(n * 8) + tb_align(n * 4) + tb_align(rows * 4) +
         2 * tb_align(rows * kTbMaxK * 8) + tb_align(rows * kTbMaxK * 4) + tb_align(rows * 4) + tb_align(rows * 8) +
         tb_align(rows * 4);
}

// Top K of the union of up to 64 lists sorted in decreasing order (lane c holds list
// c, 0 = no key; nonzero keys are unique), by one wavefront; lane r < K gets the
// r-th largest.  The K-th largest list head bounds the answer from below, so only
// the keys at or above it are ranked (one pass over them per lane); when more than
// 64 keys reach it, K rounds of a wave maximum pop the list heads instead.
// s_h: 64 entries of LDS, s_c: 64 entries of LDS (this wavefront's).
__device__ inline uint64_t merge_sorted_lists(uint64_t (&list)[kTbMaxK], int K, int lane, uint64_t* s_h,
                                              uint64_t* s_c) {
  const uint64_t head = list[0];
  s_h[lane] = head;
  wave_lds_sync();
  int g = 0;  // heads larger than this lane's (LDS reads in batches of 16)
  for (int q0 = 0; q0 < 64; q0 += 16) {
    uint64_t hq[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) hq[q] = s_h[q0 + q];
#pragma unroll
    for (int q = 0; q < 16; ++q) g += hq[q] > head ? 1 : 0;
  }
  const uint64_t tau = wave_max_u64_2step(g == K - 1 ? head : 0ull);
  int cnt = 0;
#pragma unroll
  for (int q = 0; q < kTbMaxK; ++q) cnt += (list[q] != 0ull && list[q] >= tau) ? 1 : 0;
  const int incl = wave_incl_scan_i(cnt);
  const int C = __builtin_amdgcn_readlane(incl, 63);
  uint64_t mine = 0;
  if (C <= 64) {
    const int off = incl - cnt;
#pragma unroll
    for (int q = 0; q < kTbMaxK; ++q)
      if (q < cnt) s_c[off + q] = list[q];  // a sorted list: its candidates are a prefix
    wave_lds_sync();
    const uint64_t key = lane < C ? s_c[lane] : 0ull;
    int rank = 0;
    for (int q0 = 0; q0 < C; q0 += 8) {
      uint64_t cq[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) cq[q] = s_c[q0 + q];  // (entries past C: stale keys, not counted)
#pragma unroll
      for (int q = 0; q < 8; ++q) rank += (int)((q0 + q < C) & (cq[q] > key));
    }
    wave_lds_sync();  // every lane has read the candidates
    if (lane < C && rank < K) s_c[rank] = key;
    wave_lds_sync();
    mine = lane < K && lane < C ? s_c[lane] : 0ull;
  } else {
    for (int r = 0; r < K; ++r) {
      const uint64_t w = wave_max_u64_2step(list[0]);
      if (lane == r) mine = w;
      if (w != 0ull && list[0] == w) {
#pragma unroll
        for (int q = 0; q < kTbMaxK - 1; ++q) list[q] = list[q + 1];
        list[kTbMaxK - 1] = 0ull;
      }
    }
  }
  return mine;
}

// The row's top K from its chunks' partials, by one wavefront of the row's last
// chunk workgroup: a k-way merge of the chunks' sorted lists (lane c holds chunk c's
// list in registers; keys are unique and the lane holding the maximum pops its list),
// the confidences in fp64 from the merged exp sum, and the children's values.
__device__ void tb_merge_row(const TbArgs& a, int b, int64_t rowi, int lane, uint64_t* s_h, uint64_t* s_c) {
  const int K = a.K, base = a.count[b];
  const int nd = a.frontier[rowi];
  float mc = -INFINITY;
  double sc = 0.0;
  int bc = 0;
  uint64_t list[kTbMaxK];
#pragma unroll
  for (int q = 0; q < kTbMaxK; ++q) list[q] = 0ull;
  if (lane < a.nch) {  // the other workgroups' partials: agent-scope loads
    const int64_t slot = rowi * a.nch + lane;
    mc = __uint_as_float(pub_load(reinterpret_cast<const uint32_t*>(a.ws_max) + slot));
    sc = __longlong_as_double((long long)pub_load(reinterpret_cast<const uint64_t*>(a.ws_sum) + slot));
    bc = pub_load(a.ws_bad + slot);
#pragma unroll
    for (int q = 0; q < kTbMaxK; ++q)
      if (q < K) list[q] = pub_load(a.ws_keys + slot * kTbMaxK + q);
  }
  const bool nd_in = nd >= 0 && nd < base && base <= a.cap;
  const uint64_t pp = nd_in ? a.path[(int64_t)b * a.cap + nd] : 0ull;
  const double pv = nd_in ? a.value[(int64_t)b * a.cap + nd] : 0.0;
  const bool nd_ok = nd_in && (int)(pp >> 60) < kTbMaxDepth;
  const float M = wave_max_f(mc);
  const int bad = wave_or_i(bc);
  double S = (lane < a.nch && mc > -INFINITY) ? sc * exp(((double)mc - (double)M) * a.inv_t) : 0.0;
  S = wave_sum_d(S);
  const uint64_t mine = merge_sorted_lists(list, K, lane, s_h, s_c);
  if (lane < K) {
    // confidence = softmax(row / T_d) at the child's token
    const double cf = exp(((double)tb_key_logit(mine) - (double)M) * a.inv_t) / S;
    const int64_t o = rowi * kTbMaxK + lane;
    a.row_val[o] = pv * cf;
    a.row_conf[o] = cf;
    a.row_tok[o] = tb_key_token(mine);
  }
  if (lane == 0) {
    a.row_node[rowi] = nd;
    a.row_path[rowi] = pp;
    a.row_bad[rowi] = (bad || !(M > -INFINITY) || !nd_ok) ? 1 : 0;
  }
}

template <bool kVec>
__global__ __launch_bounds__(kTbThreads) void tb_topk_kernel(TbArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t blk = blockIdx.x;
  const int c = (int)(blk % a.nch);
  const int64_t rowi = blk / a.nch;  // request * R + frontier row
  const int j = (int)(rowi % a.R), b = (int)(rowi / a.R);
  if (j >= a.fcount[b]) return;  // no node behind this row this round
  const float* src = a.logits + rowi * (int64_t)a.vocab;
  const int c0 = c * kChunk;
  // element e of a thread is token c0 + ((e >> 2) * kTbThreads + tid) * 4 + (e & 3)
  float x[kTbPer];
  if (kVec && c0 + kChunk <= a.vocab) {
#pragma unroll
    for (int k = 0; k < kTbPer / 4; ++k) {
      const tb_f32x4 f =
          __builtin_nontemporal_load(reinterpret_cast<const tb_f32x4*>(src + c0 + (k * kTbThreads + tid) * 4));
      x[4 * k + 0] = f[0];
      x[4 * k + 1] = f[1];
      x[4 * k + 2] = f[2];
      x[4 * k + 3] = f[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < kTbPer; ++e) {
      const int t = c0 + ((e >> 2) * kTbThreads + tid) * 4 + (e & 3);
      x[e] = t < a.vocab ? src[t] : -INFINITY;
    }
  }
  float lm = -INFINITY;  // this lane's maximum
  int bad = 0;
#pragma unroll
  for (int e = 0; e < kTbPer; ++e) {
    bad |= is_bad_logit(x[e]) ? 1 : 0;
    lm = fmaxf(lm, x[e]);
  }
  __shared__ float s_m[kTbThreads / 64], s_tau[kTbThreads / 64];
  __shared__ int s_b[kTbThreads / 64];
  __shared__ double s_s[kTbThreads / 64];
  __shared__ uint64_t s_k[kTbThreads / 64][kTbMaxK];
  __shared__ uint64_t s_cand[kTbCand];
  __shared__ int s_cnt;
  // Threshold: the K-th largest lane maximum of a wavefront.  At least K of its
  // tokens reach it, so no token below it is in the wavefront's top K, nor below the
  // largest such threshold in the chunk's.
  __shared__ float s_lm[kTbThreads];
  s_lm[tid] = lm;
  wave_lds_sync();
  int gl = 0;  // lane maxima of the wavefront above this lane's
  for (int q0 = 0; q0 < 64; q0 += 16) {
    float mq[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) mq[q] = s_lm[wid * 64 + q0 + q];
#pragma unroll
    for (int q = 0; q < 16; ++q) gl += mq[q] > lm ? 1 : 0;
  }
  // the K-th largest lane maximum: the largest value with at least K - 1 above it
  const float tw = wave_max_f(gl >= a.K - 1 ? lm : -INFINITY);
  const float wm = wave_max_f(lm);
  bad = wave_or_i(bad);
  if (lane == 0) {
    s_m[wid] = wm;
    s_b[wid] = bad;
    s_tau[wid] = tw;
  }
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  float cm = s_m[0], tau = s_tau[0];
  int cb = s_b[0];
#pragma unroll
  for (int w = 1; w < kTbThreads / 64; ++w) {
    cm = fmaxf(cm, s_m[w]);
    tau = fmaxf(tau, s_tau[w]);
    cb |= s_b[w];
  }
  // the chunk's exp sum, and the tokens at or above the threshold as candidates
  double acc = 0.0;
  if (cm > -INFINITY) {
#pragma unroll
    for (int e = 0; e < kTbPer; ++e) acc += (double)exp_scaled(x[e] - cm, a.es);
  }
  acc = wave_sum_d(acc);
  if (lane == 0) s_s[wid] = acc;
#pragma unroll
  for (int e = 0; e < kTbPer; ++e) {
    const int t = c0 + ((e >> 2) * kTbThreads + tid) * 4 + (e & 3);
    if (t < a.vocab && x[e] >= tau) {
      const int pos = atomicAdd(&s_cnt, 1);
      if (pos < kTbCand) s_cand[pos] = tb_key(x[e], t);
    }
  }
  __syncthreads();
  double csum = s_s[0];
#pragma unroll
  for (int w = 1; w < kTbThreads / 64; ++w) csum += s_s[w];
  const int C = s_cnt;
  const int64_t slot = rowi * a.nch + c;
  if (C <= kTbCand) {
    // the top K of the candidates by rank (keys are unique)
    if (wid == 0) {
      const uint64_t k0 = lane < C ? s_cand[lane] : 0ull, k1 = lane + 64 < C ? s_cand[lane + 64] : 0ull;
      int r0 = 0, r1 = 0;
      for (int q = 0; q < C; ++q) {
        const uint64_t kq = s_cand[q];
        r0 += kq > k0 ? 1 : 0;
        r1 += kq > k1 ? 1 : 0;
      }
      if (lane < C && r0 < a.K) pub_store(a.ws_keys + slot * kTbMaxK + r0, k0);
      if (lane + 64 < C && r1 < a.K) pub_store(a.ws_keys + slot * kTbMaxK + r1, k1);
      if (lane >= C && lane < a.K) pub_store(a.ws_keys + slot * kTbMaxK + lane, (uint64_t)0);  // fewer tokens than K
    }
  } else {
    // many tokens tie at the threshold (e.g. a row of equal logits): K rounds of a
    // wave maximum over every wavefront's keys, then over the four lists
    uint64_t key[kTbPer];
    uint64_t best = 0;
#pragma unroll
    for (int e = 0; e < kTbPer; ++e) {
      const int t = c0 + ((e >> 2) * kTbThreads + tid) * 4 + (e & 3);
      key[e] = t < a.vocab ? tb_key(x[e], t) : 0ull;
      best = key[e] > best ? key[e] : best;
    }
    for (int r = 0; r < a.K; ++r) {
      const uint64_t w = wave_max_u64(best);
      if (lane == 0) s_k[wid][r] = w;
      if (best == w) {  // the owner drops it
        best = 0;
#pragma unroll
        for (int e = 0; e < kTbPer; ++e) {
          key[e] = key[e] == w ? 0ull : key[e];
          best = key[e] > best ? key[e] : best;
        }
      }
    }
    __syncthreads();
    if (wid == 0) {
      uint64_t u = lane < 4 * a.K ? s_k[lane / a.K][lane % a.K] : 0ull;
      uint64_t mine = 0;
      for (int r = 0; r < a.K; ++r) {
        const uint64_t w = wave_max_u64(u);
        if (lane == r) mine = w;
        if (u == w) u = 0;
      }
      if (lane < a.K) pub_store(a.ws_keys + slot * kTbMaxK + lane, mine);
    }
  }
  if (tid == 0) {
    pub_store(reinterpret_cast<uint32_t*>(a.ws_max) + slot, __float_as_uint(cm));
    pub_store(reinterpret_cast<uint64_t*>(a.ws_sum) + slot, (uint64_t)__double_as_longlong(csum));
    pub_store(a.ws_bad + slot, cb);
  }
  // ---- the row's last chunk workgroup to finish merges the row ----
  __shared__ int s_last;
  stores_done();
  __syncthreads();
  if (tid == 0) s_last = pub_arrive(&a.row_cnt[rowi]) == (uint32_t)(a.nch - 1);
  __syncthreads();
  if (!s_last || wid != 0) return;
  if (lane == 0) pub_store(&a.row_cnt[rowi], 0u);
  tb_merge_row(a, b, rowi, lane, s_cand, s_cand + 64);
}

// One workgroup per request, after every row is merged: append the children (ids
// base + j * K + r: frontier order, then top-k order) and pick the next frontier.
__global__ __launch_bounds__(kTbThreads) void tb_select_kernel(TbArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = a.K;
  __shared__ double s_cv[kTbMaxFrontier * kTbMaxK];
  __shared__ double s_cc[kTbMaxFrontier * kTbMaxK];
  __shared__ int s_ct[kTbMaxFrontier * kTbMaxK];
  __shared__ int s_fr[kTbMaxFrontier];
  __shared__ uint64_t s_pp[kTbMaxFrontier];
  __shared__ int s_err;
  const int fc = a.fcount[b], base = a.count[b];
  if (fc == 0) return;  // this request is finished (or failed earlier)
  if (fc < 0 || fc > a.R || base < 1 || base > a.cap || fc * K > a.cap - base) {
    if (tid == 0) {
      report(a.status, SPEC_ERR_BAD_INPUT);
      a.fcount[b] = 0;
    }
    return;
  }
  if (tid == 0) s_err = 0;
  __syncthreads();
  const int nnew = fc * K;
  for (int i = tid; i < nnew; i += kTbThreads) {
    const int j = i / K, r = i - j * K;
    const int64_t o = ((int64_t)b * a.R + j) * kTbMaxK + r;
    s_cv[i] = a.row_val[o];
    s_cc[i] = a.row_conf[o];
    s_ct[i] = a.row_tok[o];
  }
  if (tid < fc) {
    const int64_t rowi = (int64_t)b * a.R + tid;
    s_fr[tid] = a.row_node[rowi];
    s_pp[tid] = a.row_path[rowi];
    if (a.row_bad[rowi]) s_err = 1;
  }
  __syncthreads();
  if (s_err) {
    if (tid == 0) {
      report(a.status, SPEC_ERR_BAD_INPUT);
      a.fcount[b] = 0;
    }
    return;
  }
  for (int i = tid; i < nnew; i += kTbThreads) {
    const int jj = i / K, r = i - jj * K;
    const int64_t o = (int64_t)b * a.cap + base + i;
    const uint64_t pp = s_pp[jj];
    const int d = (int)(pp >> 60) + 1;
    a.parent[o] = s_fr[jj];
    a.token[o] = s_ct[i];
    a.value[o] = s_cv[i];
    a.conf[o] = s_cc[i];
    a.path[o] = ((uint64_t)d << 60) | (pp & ((1ull << 60) - 1)) | ((uint64_t)r << (60 - 4 * d));
  }
  // the next frontier: the select_k new children of largest value (ties to the lower
  // id), each child ranked against all new children by its own thread (branch-free
  // comparisons over broadcast LDS reads).  Best-first: tb_frontier_kernel picks it.
  const int sk = min(a.select_k, nnew);
  if (a.policy == 0 && tid < nnew) {
    const double v = s_cv[tid];
    int rank = 0;
    for (int q0 = 0; q0 < nnew; q0 += 8) {
      double vq[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) vq[q] = s_cv[min(q0 + q, nnew - 1)];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = q0 + q;
        rank += (int)((i < nnew) & ((vq[q] > v) | ((vq[q] == v) & (i < tid))));
      }
    }
    if (rank < sk) a.frontier[(int64_t)b * a.R + rank] = base + tid;
  }
  if (tid == 0) {
    a.fcount[b] = sk;
    a.count[b] = base + nnew;
  }
}

// Best-first policy, after the children are appended: the next frontier is the
// select_k leaves of largest value (ties to the lower id) among every node of the
// request that has no children and sits above the depth limit.  One thread per node,
// a bitonic sort as in the rerank.
__global__ __launch_bounds__(kTbMaxCap) void tb_frontier_kernel(TbArgs a) {
  __shared__ int s_kid[kTbMaxCap];
  __shared__ double s_v[kTbMaxCap];
  __shared__ uint32_t s_t[kTbMaxCap];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (a.fcount[b] == 0) return;  // finished, failed, or refused this round
  const int cnt = a.count[b];
  if (cnt < 1 || cnt > a.cap) return;  // (the select kernel has refused such a state)
  const int64_t cb = (int64_t)b * a.cap;
  s_kid[tid] = 0;
  __syncthreads();
  if (tid >= 1 && tid < cnt) {
    const int p = a.parent[cb + tid];
    if (p >= 0 && p < cnt) s_kid[p] = 1;
  }
  __syncthreads();
  const bool leaf = tid < cnt && !s_kid[tid] && (int)(a.path[cb + tid] >> 60) < kTbMaxDepth;
  double v = leaf ? a.value[cb + tid] : -1.0;  // values are >= 0: non-leaves sort last
  uint32_t t = leaf ? (uint32_t)tid : 0xffffffffu;
  const int n_leaves = __syncthreads_count(leaf);
  int P = 2;
  while (P < cnt) P <<= 1;
  for (int k = 2; k <= P; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      double pv;
      uint32_t pt;
      if (jj < 64) {
        pv = __shfl_xor(v, jj);
        pt = (uint32_t)__shfl_xor((int)t, jj);
      } else {
        s_v[tid] = v;
        s_t[tid] = t;
        __syncthreads();
        pv = s_v[tid ^ jj];
        pt = s_t[tid ^ jj];
        __syncthreads();
      }
      const bool keep_first = ((tid & k) == 0) == ((tid & jj) == 0);
      const bool partner_first = rr_before(pv, pt, v, t);
      if (partner_first == keep_first) {
        v = pv;
        t = pt;
      }
    }
  const int sk = min(a.select_k, n_leaves);
  if (tid < sk) a.frontier[(int64_t)b * a.R + tid] = (int)t;
  if (tid == 0) a.fcount[b] = sk;
}

__global__ void tb_init_kernel(const int32_t* root_token, int32_t batch, int32_t cap, int32_t R, int32_t* parent,
                               int32_t* token, uint64_t* path, double* value, double* conf, int32_t* count,
                               int32_t* frontier, int32_t* fcount) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int64_t o = (int64_t)b * cap;
  parent[o] = -1;
  token[o] = root_token[b];
  path[o] = 0;
  value[o] = 1.0;
  conf[o] = 1.0;
  count[b] = 1;
  frontier[(int64_t)b * R] = 0;
  fcount[b] = 1;
}

struct RrArgs {
  const int32_t *parent, *token;
  const uint64_t* path;
  const double* value;
  const int32_t* count;
  int32_t cap, n_final;
  int32_t *out_parent, *out_token, *out_n, *out_id, *status;
};


// Bitonic sort of the candidates, one per thread: exchanges within a wavefront go
// through lane shuffles, the longer ones through LDS.
__global__ __launch_bounds__(kTbRerankThreads) void tb_rerank_kernel(RrArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __shared__ double s_v[kTbMaxCap];
  __shared__ uint32_t s_t[kTbMaxCap];
  __shared__ int s_pos[kTbMaxCap];
  __shared__ uint64_t s_key[64];
  __shared__ int s_sel[64];
  const int cnt = a.count[b];
  const int64_t ob = (int64_t)b * a.n_final;
  if (cnt < 1 || cnt > a.cap) {  // no tree to rank
    for (int i = tid; i < a.n_final; i += kTbRerankThreads) {
      a.out_parent[ob + i] = -1;
      a.out_token[ob + i] = -1;
      a.out_id[ob + i] = -1;
    }
    if (tid == 0) {
      a.out_n[b] = 0;
      report(a.status, SPEC_ERR_BAD_INPUT);
    }
    return;
  }
  const int m = cnt - 1;  // candidates besides the root
  int P = 2;
  while (P < m) P <<= 1;
  const int64_t cb = (int64_t)b * a.cap;
  double v = -1.0;  // padding sorts last: values are >= 0
  uint32_t t = 0xffffffffu;
  if (tid < m) {
    const int id = tid + 1;
    v = a.value[cb + id];
    t = ((uint32_t)(a.path[cb + id] >> 60) << 10) | (uint32_t)id;
  }
  for (int k = 2; k <= P; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      double pv;
      uint32_t pt;
      if (jj < 64) {
        pv = __shfl_xor(v, jj);
        pt = (uint32_t)__shfl_xor((int)t, jj);
      } else {
        s_v[tid] = v;
        s_t[tid] = t;
        __syncthreads();
        pv = s_v[tid ^ jj];
        pt = s_t[tid ^ jj];
        __syncthreads();
      }
      // in a rising run the lower index keeps the earlier element, in a falling run the later
      const bool keep_first = ((tid & k) == 0) == ((tid & jj) == 0);
      const bool partner_first = rr_before(pv, pt, v, t);
      if (partner_first == keep_first) {
        v = pv;
        t = pt;
      }
    }
  const int n = min(a.n_final - 1, m) + 1;  // the root and the top n - 1
  if (tid < n - 1) s_t[tid] = t;
  __syncthreads();
  if (wid != 0) return;
  // breadth-first order by path key
  int id = -1;
  uint64_t key = ~0ull;
  if (lane < n) {
    id = lane == 0 ? 0 : (int)(s_t[lane - 1] & 0x3ffu);
    if (id >= cnt) id = 0;  // (only with values that do not order, e.g. NaN: caught below as a repeated key)
    key = a.path[cb + id];
  }
  s_key[lane] = key;
  s_sel[lane] = -1;
  wave_lds_sync();
  int rank = 0;
  for (int q = 0; q < n; ++q) rank += s_key[q] < key ? 1 : 0;
  if (lane < n) {
    s_sel[rank] = id;
    s_pos[id] = rank;
  }
  wave_lds_sync();
  int bad = 0;
  if (lane < n) {
    int idr = s_sel[lane];
    int pf = -1;
    if (idr < 0 || idr >= cnt) {  // two kept nodes with one path key: the state is not a valid tree
      bad = 1;
      idr = 0;
    } else if (lane > 0) {
      const int pp = a.parent[cb + idr];
      const int pr = (pp >= 0 && pp < cnt) ? s_pos[pp] : -1;
      if (pr >= 0 && pr < lane && s_sel[pr] == pp)
        pf = pr;
      else
        bad = 1;  // a kept node whose parent was not kept: the state is not a valid tree
    }
    a.out_parent[ob + lane] = pf;
    a.out_token[ob + lane] = a.token[cb + idr];
    a.out_id[ob + lane] = idr;
  } else if (lane < a.n_final) {
    a.out_parent[ob + lane] = -1;
    a.out_token[ob + lane] = -1;
    a.out_id[ob + lane] = -1;
  }
  bad = wave_or_i(bad);
  if (lane == 0) {
    a.out_n[b] = bad ? 0 : n;
    if (bad) report(a.status, SPEC_ERR_BAD_TREE);
  }
}

inline int tb_chunks(int32_t vocab) { return (vocab + kChunk - 1) / kChunk; }

}  // namespace spectree

extern "C" int spec_tree_build_init(const int32_t* root_token, int32_t batch, int32_t cap, int32_t max_frontier,
                                    int32_t* cand_parent, int32_t* cand_token, uint64_t* cand_path,
                                    double* cand_value, double* cand_conf, int32_t* cand_count, int32_t* frontier,
                                    int32_t* frontier_count, void* stream) {
  using namespace spectree;
  if (!root_token || !cand_parent || !cand_token || !cand_path || !cand_value || !cand_conf || !cand_count ||
      !frontier || !frontier_count)
    return SPEC_ERR_INVALID_ARG;
  if (batch < 1 || cap < 1 || cap > kTbMaxCap || max_frontier < 1 || max_frontier > kTbMaxFrontier)
    return SPEC_ERR_INVALID_ARG;
  hipLaunchKernelGGL(tb_init_kernel, dim3((unsigned)((batch + 63) / 64)), dim3(64), 0, (hipStream_t)stream,
                     root_token, batch, cap, max_frontier, cand_parent, cand_token, cand_path, cand_value, cand_conf,
                     cand_count, frontier, frontier_count);
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}

extern "C" size_t spec_tree_expand_workspace_size(int32_t batch, int32_t max_frontier, int32_t vocab) {
  using namespace spectree;
  if (batch < 1 || max_frontier < 1 || max_frontier > kTbMaxFrontier || vocab < 1 ||
      vocab > kTbMaxChunks * kChunk)
    return 0;
  return tb_ws_bytes(batch, max_frontier, tb_chunks(vocab));
}

extern "C" int spec_tree_expand(const float* draft_logits, int32_t vocab, float T_d, int32_t batch,
                                int32_t max_frontier, int32_t top_k, int32_t select_k, int32_t policy, int32_t cap,
                                int32_t* cand_parent, int32_t* cand_token, uint64_t* cand_path, double* cand_value,
                                double* cand_conf, int32_t* cand_count, int32_t* frontier, int32_t* frontier_count,
                                void* workspace, size_t workspace_bytes, int32_t* status, void* stream) {
  using namespace spectree;
  if (!draft_logits || !cand_parent || !cand_token || !cand_path || !cand_value || !cand_conf || !cand_count ||
      !frontier || !frontier_count)
    return SPEC_ERR_INVALID_ARG;
  if (batch < 1 || max_frontier < 1 || max_frontier > kTbMaxFrontier || top_k < 1 || top_k > kTbMaxK ||
      select_k < 1 || select_k > max_frontier || cap < 1 || cap > kTbMaxCap || vocab < top_k ||
      (policy != 0 && policy != 1))
    return SPEC_ERR_INVALID_ARG;
  if (!(T_d > 0.0f) || !isfinite(T_d)) return SPEC_ERR_INVALID_ARG;
  if (vocab > kTbMaxChunks * kChunk) return SPEC_ERR_UNSUPPORTED;
  const int nch = tb_chunks(vocab);
  const size_t need = tb_ws_bytes(batch, max_frontier, nch);
  if (!workspace || workspace_bytes < need) return SPEC_ERR_WORKSPACE;
  const int64_t blocks = (int64_t)batch * max_frontier * nch;
  if (blocks > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  TbArgs a;
  a.logits = draft_logits;
  a.vocab = vocab;
  a.nch = nch;
  a.R = max_frontier;
  a.K = top_k;
  a.select_k = select_k;
  a.policy = policy;
  a.cap = cap;
  a.inv_t = 1.0 / (double)T_d;
  a.es = make_exp_scale(a.inv_t);
  a.parent = cand_parent;
  a.token = cand_token;
  a.path = cand_path;
  a.value = cand_value;
  a.conf = cand_conf;
  a.count = cand_count;
  a.frontier = frontier;
  a.fcount = frontier_count;
  const size_t n = (size_t)batch * max_frontier * nch;
  char* w = (char*)workspace;
  a.ws_keys = (uint64_t*)w;
  w += tb_align(n * kTbMaxK * 8);
  a.ws_max = (float*)w;
  w += tb_align(n * 4);
  a.ws_sum = (double*)w;
  w += tb_align(n * 8);
  a.ws_bad = (int32_t*)w;
  w += tb_align(n * 4);
  const size_t rows = (size_t)batch * max_frontier;
  a.row_cnt = (uint32_t*)w;
  w += tb_align(rows * 4);
  a.row_val = (double*)w;
  w += tb_align(rows * kTbMaxK * 8);
  a.row_conf = (double*)w;
  w += tb_align(rows * kTbMaxK * 8);
  a.row_tok = (int32_t*)w;
  w += tb_align(rows * kTbMaxK * 4);
  a.row_node = (int32_t*)w;
  w += tb_align(rows * 4);
  a.row_path = (uint64_t*)w;
  w += tb_align(rows * 8);
  a.row_bad = (int32_t*)w;
  a.status = status;
  hipStream_t st = (hipStream_t)stream;
  const bool vec = vocab % 4 == 0 && (((uintptr_t)draft_logits & 15) == 0);
  if (vec)
    hipLaunchKernelGGL(tb_topk_kernel<true>, dim3((unsigned)blocks), dim3(kTbThreads), 0, st, a);
  else
    hipLaunchKernelGGL(tb_topk_kernel<false>, dim3((unsigned)blocks), dim3(kTbThreads), 0, st, a);
  SPEC_LAUNCH_CHECK();
  hipLaunchKernelGGL(tb_select_kernel, dim3((unsigned)batch), dim3(kTbThreads), 0, st, a);
  SPEC_LAUNCH_CHECK();
  if (policy == 1) {
    hipLaunchKernelGGL(tb_frontier_kernel, dim3((unsigned)batch), dim3(kTbMaxCap), 0, st, a);
    SPEC_LAUNCH_CHECK();
  }
  return SPEC_OK;
}

extern "C" int spec_tree_rerank(const int32_t* cand_parent, const int32_t* cand_token, const uint64_t* cand_path,
                                const double* cand_value, const int32_t* cand_count, int32_t batch, int32_t cap,
                                int32_t n_final, int32_t* parent, int32_t* tokens, int32_t* n_nodes,
                                int32_t* cand_id, int32_t* status, void* stream) {
  using namespace spectree;
  if (!cand_parent || !cand_token || !cand_path || !cand_value || !cand_count || !parent || !tokens || !n_nodes ||
      !cand_id)
    return SPEC_ERR_INVALID_ARG;
  if (batch < 1 || cap < 1 || cap > kTbMaxCap || n_final < 1 || n_final > 64) return SPEC_ERR_INVALID_ARG;
  RrArgs a;
  a.parent = cand_parent;
  a.token = cand_token;
  a.path = cand_path;
  a.value = cand_value;
  a.count = cand_count;
  a.cap = cap;
  a.n_final = n_final;
  a.out_parent = parent;
  a.out_token = tokens;
  a.out_n = n_nodes;
  a.out_id = cand_id;
  a.status = status;
  hipLaunchKernelGGL(tb_rerank_kernel, dim3((unsigned)batch), dim3(kTbRerankThreads), 0, (hipStream_t)stream, a);
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}
