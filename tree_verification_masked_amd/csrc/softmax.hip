// Per-node vocabulary softmax statistics.
//
// "The EAGLE Family" (consciousengines.com), "Why predict features instead of
// tokens?": the next-token distribution is the softmax of the LM-head output.
// Tree-verification notes, parts A and D.2: one softmax per tree node, N x |V|
// elements per verify, bound by memory bandwidth.
//
// One pass over the logits.  A row is cut into chunks of kChunk tokens; each
// workgroup reads one chunk with 16-byte loads that are all in flight at once
// (full chunks take a branch-free path), keeps it in registers, and writes the
// chunk's maximum m_c, first argmax and s_c = sum exp((l - m_c) / T) accumulated in
// fp64.  A second, small launch merges the chunk partials of each row in chunk
// order:  m = max_c m_c,  Z = sum_c s_c exp((m_c - m) / T).  (Merging inside the
// first launch would make every workgroup wait for its partials to become visible
// device-wide before signalling; on MI355X that costs more than the extra launch.)
// One launch can cover two logit arrays (target and draft rows, each with its own
// temperature).
#include "attn_combine.hpp"
#include "greedy_walk.hpp"
#include "internal.hpp"

namespace spectree {

constexpr int kSmThreads = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kSmPerThread = kChunk / kSmThreads;  // 32 fp32 elements held per thread

inline int sm_chunks(int32_t vocab) { return (vocab + kChunk - 1) / kChunk; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct SmSet {
  const float* logits;
  int64_t rows;
  double inv_t;
  ExpScale es;
  int greedy;
  float* row_max;
  float* row_sumexp;
  int32_t* row_argmax;
  float* cmax;      // [rows, nch]  chunk maxima (caller's array or workspace)
  double* csum;     // [rows, nch]  chunk sums of exp((l - m_c)/T)
  int32_t* carg;    // [rows, nch]  workspace
  int32_t* cbad;    // [rows, nch]  workspace
  // draft rows of a step given its tree: only the rows of nodes with children are
  // needed (a leaf's draft row takes no part; tree notes, parts C and G)
  const int32_t* parent;   // [batch, n_max] or null
  const int32_t* n_nodes;  // [batch]
  int32_t n_max;
};

// Workspace of one logit array: argmax / bad flags per chunk, and the chunk maxima
// and sums unless the caller asked for them.
inline size_t sm_set_bytes(int64_t rows, int32_t vocab) {
  const size_t n = (size_t)rows * (size_t)sm_chunks(vocab);
  return align256(n * 4) * 3 + align256(n * 8);
}
inline void sm_set_carve(char* base, int64_t rows, int32_t vocab, SmSet* s, float* cmax, double* csum) {
  const size_t n = (size_t)rows * (size_t)sm_chunks(vocab);
  size_t off = 0;
  s->carg = (int32_t*)(base + off);
  off += align256(n * 4);
  s->cbad = (int32_t*)(base + off);
  off += align256(n * 4);
  s->cmax = cmax ? cmax : (float*)(base + off);
  off += align256(n * 4);
  s->csum = csum ? csum : (double*)(base + off);
}

__device__ inline void better(float& m, int& a, float om, int oa) {
  if (om > m || (om == m && oa < a)) {
    m = om;
    a = oa;
  }
}
// Wave-wide (max, lowest index) in DPP steps; every lane gets the result.
template <int kCtrl, int kRowMask = 0xf>
__device__ inline void better_dpp(float& m, int& a) {
  const float m2 = dpp_f<kCtrl, kRowMask>(m, m);
  const int a2 = dpp_i<kCtrl, kRowMask>(a, a);
  better(m, a, m2, a2);
}
__device__ inline void wave_best(float& m, int& a) {
  better_dpp<kDppQuad1032>(m, a);
  better_dpp<kDppQuad2301>(m, a);
  better_dpp<kDppHalfMirror>(m, a);
  better_dpp<kDppMirror>(m, a);
  better_dpp<kDppBcast15, 0xa>(m, a);
  better_dpp<kDppBcast31, 0xc>(m, a);
  m = lane63_f(m);
  a = lane63_i(a);
}

// kCombD > 0: the workgroups after the chunks finish an attention call's split
// combine (head size kCombD, element type CombT), one output row per wave.
template <bool kVec, int kCombD, typename CombT>
__global__ __launch_bounds__(kSmThreads) void softmax_stats_kernel(SmSet A, SmSet B, int32_t vocab, int nch,
                                                                   int32_t* status, AttnArgs comb_args, CombT* comb_out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  int64_t blk = blockIdx.x;
  // Workgroup order with a second set: its rows, then the split combine's rows, then
  // the first set's rows.  Given the tree, a second-set workgroup reads the parent
  // links before its row, and the combine reads partials another launch wrote; both
  // waits overlap the first set's streaming behind them.  With one set the combine's
  // rows come after it.
  const int64_t blocks_a = A.rows * nch, blocks_b = B.rows * nch;
  const int64_t blocks_c = (int64_t)gridDim.x - blocks_a - blocks_b;  // the combine's (0 without it)
  const int64_t c_begin = blocks_b > 0 ? blocks_b : blocks_a;
  if constexpr (kCombD > 0) {
    if (blk >= c_begin && blk < c_begin + blocks_c) {
      // four splits per load round: the chunk workgroups' register budget
      attn_combine_row<kCombD, CombT, 4>(comb_args, comb_out, (blk - c_begin) * 4 + wid);
      return;
    }
  }
  const bool second = blk < blocks_b;
  const SmSet& S = second ? B : A;
  if (!second) blk -= blocks_b + (kCombD > 0 && blocks_b > 0 ? blocks_c : 0);
  const int chunk = (int)(blk % nch);
  const int64_t row = blk / nch;
  if (S.parent) {  // a node without children (or a padding slot): its row is not needed
    const int64_t b = row / S.n_max;
    const int n = (int)(row % S.n_max), nb = S.n_nodes[b];
    const int par = lane < S.n_max ? S.parent[b * S.n_max + lane] : -2;
    if (n >= nb || !__ballot(lane > n && lane < nb && par == n)) return;  // the same in every wave
  }
  const float* src = S.logits + row * (int64_t)vocab;
  const int c0 = chunk * kChunk;

  // Element (k, v) of a thread is token c0 + (k * kSmThreads + tid) * 4 + v, so
  // consecutive threads read consecutive 16-byte pieces.
  float x[kSmPerThread];
  if (kVec && c0 + kChunk <= vocab) {
#pragma unroll
    for (int k = 0; k < kSmPerThread / 4; ++k) {
      // streaming, read-once data: non-temporal loads
      const f32x4 f4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + c0 + (k * kSmThreads + tid) * 4));
      const float4 f = make_float4(f4[0], f4[1], f4[2], f4[3]);
      x[4 * k + 0] = f.x;
      x[4 * k + 1] = f.y;
      x[4 * k + 2] = f.z;
      x[4 * k + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kSmPerThread / 4; ++k)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = c0 + (k * kSmThreads + tid) * 4 + v;
        x[4 * k + v] = t < vocab ? src[t] : -INFINITY;
      }
  }
  float m = -INFINITY;
  int am = 0x7fffffff;
  int bad = 0;
#pragma unroll
  for (int k = 0; k < kSmPerThread / 4; ++k)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float e = x[4 * k + v];
      bad |= is_bad_logit(e) ? 1 : 0;
      if (e > m) {  // a thread visits its tokens in increasing order
        m = e;
        am = c0 + (k * kSmThreads + tid) * 4 + v;
      }
    }
  __shared__ float s_m[kSmThreads / 64];
  __shared__ int s_a[kSmThreads / 64];
  __shared__ int s_b[kSmThreads / 64];
  __shared__ double s_s[kSmThreads / 64];
  wave_best(m, am);
  bad = wave_or_i(bad);
  if (lane == 0) {
    s_m[wid] = m;
    s_a[wid] = am;
    s_b[wid] = bad;
  }
  __syncthreads();
  float cm = s_m[0];
  int ca = s_a[0];
  int cb = s_b[0];
#pragma unroll
  for (int w = 1; w < kSmThreads / 64; ++w) {
    better(cm, ca, s_m[w], s_a[w]);
    cb |= s_b[w];
  }
  double csum = 0.0;
  if (!S.greedy && cm > -INFINITY) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kSmPerThread; ++k) acc += (double)exp_scaled(x[k] - cm, S.es);
    acc = wave_sum_d(acc);
    if (lane == 0) s_s[wid] = acc;
    __syncthreads();
    csum = s_s[0];
#pragma unroll
    for (int w = 1; w < kSmThreads / 64; ++w) csum += s_s[w];
  }
  if (tid == 0) {
    const int64_t slot = row * nch + chunk;
    S.cmax[slot] = cb ? NAN : cm;  // an invalid chunk is marked in its maximum too
    if (cb) report(status, SPEC_ERR_BAD_INPUT);
    S.csum[slot] = csum;
    S.carg[slot] = ca;
    S.cbad[slot] = cb;
  }
}

// One wavefront per row: merge the chunk partials in chunk order.  With a walk (g),
// the rows of A are a batch of requests' node rows at T = 0: the wave that merges a
// request's last row (an arrival on req_count, which it leaves at zero) then runs
// that request's greedy walk.
__global__ __launch_bounds__(256) void softmax_merge_kernel(SmSet A, SmSet B, int nch, int32_t* status, GreedyArgs g,
                                                            uint32_t* req_count) {
  const int lane = threadIdx.x & 63;
  int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= A.rows + B.rows) return;
  const bool second = row >= A.rows;
  const SmSet& S = second ? B : A;
  if (second) row -= A.rows;
  // the first 64 chunks' partials are loaded in one round (lane c holds chunk c)
  const int c0 = min(lane, nch - 1);
  const float mc0 = S.cmax[row * nch + c0];
  const int ac0 = S.carg[row * nch + c0], bc0 = S.cbad[row * nch + c0];
  const double sc0 = S.greedy ? 0.0 : S.csum[row * nch + c0];
  float m_all = -INFINITY;
  int a_all = 0x7fffffff;
  int b_all = 0;
  if (lane < nch) {
    better(m_all, a_all, mc0, ac0);
    b_all = bc0;
  }
  for (int c = lane + 64; c < nch; c += 64) {
    better(m_all, a_all, S.cmax[row * nch + c], S.carg[row * nch + c]);
    b_all |= S.cbad[row * nch + c];
  }
  wave_best(m_all, a_all);
  b_all = wave_or_i(b_all);
  double z = 0.0;
  if (!S.greedy && m_all > -INFINITY) {
    if (lane < nch && mc0 > -INFINITY) z = sc0 * exp(((double)mc0 - (double)m_all) * S.inv_t);
    for (int c = lane + 64; c < nch; c += 64) {
      const float mc = S.cmax[row * nch + c];
      if (mc > -INFINITY) z += S.csum[row * nch + c] * exp(((double)mc - (double)m_all) * S.inv_t);
    }
    z = wave_sum_d(z);
  }
  if (lane == 0) {
    // agent-scope stores: a walk in this launch (below) may read them from another XCD,
    // whose L2 a plain store does not reach
    const bool bad_row = b_all || !(m_all > -INFINITY);
    pub_store(&S.row_max[row], bad_row ? NAN : m_all);
    if (S.row_sumexp) pub_store(&S.row_sumexp[row], bad_row ? NAN : (float)z);
    if (S.row_argmax) pub_store(&S.row_argmax[row], bad_row ? -1 : a_all);
    if (bad_row) report(status, SPEC_ERR_BAD_INPUT);
  }
  if (g.accepted_child && !second) {
    const int b = (int)(row / g.n_max);
    int last = 0;
    if (lane == 0) {
      stores_done();
      last = pub_arrive(&req_count[b]) == (uint32_t)(g.n_max - 1);
    }
    if (__shfl(last, 0)) {
      if (lane == 0) pub_store(&req_count[b], 0u);
      greedy_walk_wave<true>(g, b);
    }
  }
}

// probs[r, x] = exp((l - m) / T) / Z, tests only.
__global__ __launch_bounds__(256) void softmax_probs_kernel(const float* __restrict__ logits, int32_t vocab,
                                                            ExpScale es, const float* __restrict__ row_max,
                                                            const float* __restrict__ row_sumexp,
                                                            float* __restrict__ probs) {
  const int64_t row = blockIdx.y;
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= vocab) return;
  const float m = row_max[row];
  const float inv_z = 1.0f / row_sumexp[row];
  const float l = logits[row * (int64_t)vocab + x];
  probs[row * (int64_t)vocab + x] = isnan(m) ? NAN : exp_scaled(l - m, es) * inv_z;
}

inline SmSet make_set(const float* logits, int64_t rows, float t, float* mx, float* se, int32_t* am) {
  SmSet s{};
  s.logits = logits;
  s.rows = rows;
  s.greedy = t == 0.0f;
  s.inv_t = s.greedy ? 0.0 : 1.0 / (double)t;
  s.es = make_exp_scale(s.inv_t);
  s.row_max = mx;
  s.row_sumexp = se;
  s.row_argmax = am;
  return s;
}

// The chunk pass (followed, in the same launch, by the rows of `comb` when given),
// then (merge) the row merge.
inline int launch_stats(const SmSet& A, const SmSet& B, int32_t vocab, int32_t* status, hipStream_t st,
                        bool merge, const AttnCombine* comb, const GreedyArgs* walk = nullptr,
                        uint32_t* req_count = nullptr) {
  const int nch = sm_chunks(vocab);
  AttnCombine c{};
  if (comb) c = *comb;
  const int64_t blocks = (A.rows + B.rows) * nch + (c.rows + 3) / 4;
  if (blocks * kSmThreads > 0xffffffffLL) return SPEC_ERR_UNSUPPORTED;  // a dispatch counts work-items in 32 bits
  bool vec = vocab % 4 == 0 && (((uintptr_t)A.logits & 15) == 0);
  if (B.rows) vec = vec && (((uintptr_t)B.logits & 15) == 0);
  const dim3 g((unsigned)blocks), blk(kSmThreads);
  // the instance without the combine rows keeps the plain pass's registers
  const int form = c.rows <= 0 ? 0 : c.dtype == SPEC_BF16 ? (c.head_dim == 128 ? 1 : 2) : (c.head_dim == 128 ? 3 : 4);
  if (vec) {
    switch (form) {
      case 0: hipLaunchKernelGGL((softmax_stats_kernel<true, 0, float>), g, blk, 0, st, A, B, vocab, nch, status, c.a, (float*)nullptr); break;
      case 1: hipLaunchKernelGGL((softmax_stats_kernel<true, 128, __bf16>), g, blk, 0, st, A, B, vocab, nch, status, c.a, (__bf16*)c.out); break;
      case 2: hipLaunchKernelGGL((softmax_stats_kernel<true, 64, __bf16>), g, blk, 0, st, A, B, vocab, nch, status, c.a, (__bf16*)c.out); break;
      case 3: hipLaunchKernelGGL((softmax_stats_kernel<true, 128, float>), g, blk, 0, st, A, B, vocab, nch, status, c.a, (float*)c.out); break;
      default: hipLaunchKernelGGL((softmax_stats_kernel<true, 64, float>), g, blk, 0, st, A, B, vocab, nch, status, c.a, (float*)c.out); break;
    }
  } else {
    switch (form) {
      case 0: hipLaunchKernelGGL((softmax_stats_kernel<false, 0, float>), g, blk, 0, st, A, B, vocab, nch, status, c.a, (float*)nullptr); break;
      case 1: hipLaunchKernelGGL((softmax_stats_kernel<false, 128, __bf16>), g, blk, 0, st, A, B, vocab, nch, status, c.a, (__bf16*)c.out); break;
      case 2: hipLaunchKernelGGL((softmax_stats_kernel<false, 64, __bf16>), g, blk, 0, st, A, B, vocab, nch, status, c.a, (__bf16*)c.out); break;
      case 3: hipLaunchKernelGGL((softmax_stats_kernel<false, 128, float>), g, blk, 0, st, A, B, vocab, nch, status, c.a, (float*)c.out); break;
      default: hipLaunchKernelGGL((softmax_stats_kernel<false, 64, float>), g, blk, 0, st, A, B, vocab, nch, status, c.a, (float*)c.out); break;
    }
  }
  SPEC_LAUNCH_CHECK();
  if (!merge) return SPEC_OK;  // invalid rows were reported by the chunk pass
  const int64_t rows = A.rows + B.rows;
  GreedyArgs wk{};
  if (walk) wk = *walk;
  hipLaunchKernelGGL(softmax_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, A, B, nch, status, wk,
                     req_count);
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}

}  // namespace spectree

extern "C" int32_t spec_tree_softmax_chunk(void) { return spectree::kChunk; }

extern "C" size_t spec_tree_softmax_workspace_size(int64_t rows, int32_t vocab) {
  if (rows < 1 || vocab < 1) return 0;
  return spectree::sm_set_bytes(rows, vocab);
}

namespace spectree {
int softmax_call(const float* logits, int64_t rows, int32_t vocab, float temperature, float* row_max,
                 float* row_sumexp, int32_t* row_argmax, float* probs, float* chunk_max, double* chunk_sum,
                 void* workspace, size_t workspace_bytes, int32_t* status, void* stream, const AttnCombine* comb,
                 const GreedyArgs* walk, uint32_t* req_count) {
  if (!logits || !row_max || rows < 1 || vocab < 1) return SPEC_ERR_INVALID_ARG;
  if (!(temperature >= 0.0f) || isinf(temperature)) return SPEC_ERR_INVALID_ARG;
  const bool greedy = temperature == 0.0f;
  if (!greedy && !row_sumexp) return SPEC_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < sm_set_bytes(rows, vocab)) return SPEC_ERR_WORKSPACE;
  SmSet A = make_set(logits, rows, temperature, row_max, row_sumexp, row_argmax);
  sm_set_carve((char*)workspace, rows, vocab, &A, chunk_max, chunk_sum);
  SmSet B{};
  const int rc = launch_stats(A, B, vocab, status, (hipStream_t)stream, true, comb, walk, req_count);
  if (rc != SPEC_OK) return rc;
  if (probs && !greedy) {
    if (rows > 65535) return SPEC_ERR_UNSUPPORTED;
    dim3 g2((unsigned)((vocab + 255) / 256), (unsigned)rows);
    hipLaunchKernelGGL(softmax_probs_kernel, g2, dim3(256), 0, (hipStream_t)stream, logits, vocab, A.es, row_max,
                       row_sumexp, probs);
    SPEC_LAUNCH_CHECK();
  }
  return SPEC_OK;
}
}  // namespace spectree

extern "C" int spec_tree_softmax(const float* logits, int64_t rows, int32_t vocab, float temperature,
                                 float* row_max, float* row_sumexp, int32_t* row_argmax, float* probs,
                                 float* chunk_max, double* chunk_sum, void* workspace, size_t workspace_bytes,
                                 int32_t* status, void* stream) {
  return spectree::softmax_call(logits, rows, vocab, temperature, row_max, row_sumexp, row_argmax, probs, chunk_max,
                                chunk_sum, workspace, workspace_bytes, status, stream, nullptr, nullptr, nullptr);
}

namespace spectree {
size_t softmax_pair_counters_offset(int64_t rows, int32_t vocab) { return 2 * sm_set_bytes(rows, vocab); }
}  // namespace spectree

extern "C" size_t spec_tree_softmax_pair_workspace_size(int64_t rows, int32_t vocab) {
  if (rows < 1 || vocab < 1) return 0;
  // two row sets, then the verification step's per-request counters at T = 0
  return 2 * spectree::sm_set_bytes(rows, vocab) + spectree::align256((size_t)rows * 4);
}

namespace spectree {
int softmax_pair_call(const float* tgt_logits, float temperature, const float* dft_logits, float draft_temperature,
                      int64_t rows, int32_t vocab, const int32_t* parent, const int32_t* n_nodes, int32_t n_max,
                      float* tgt_max, float* tgt_sumexp, int32_t* tgt_argmax, float* tgt_chunk_max,
                      double* tgt_chunk_sum, float* dft_max, float* dft_sumexp, float* dft_chunk_max,
                      double* dft_chunk_sum, void* workspace, size_t workspace_bytes, int32_t* status, void* stream,
                      const AttnCombine* comb) {
  if (!tgt_logits || !dft_logits) return SPEC_ERR_INVALID_ARG;
  const bool row_out = tgt_max || tgt_sumexp || dft_max || dft_sumexp;
  if (row_out && !(tgt_max && tgt_sumexp && dft_max && dft_sumexp)) return SPEC_ERR_INVALID_ARG;  // all or none
  if ((tgt_chunk_max == nullptr) != (tgt_chunk_sum == nullptr)) return SPEC_ERR_INVALID_ARG;
  if ((dft_chunk_max == nullptr) != (dft_chunk_sum == nullptr)) return SPEC_ERR_INVALID_ARG;
  if (!row_out && (!tgt_chunk_max || !dft_chunk_max)) return SPEC_ERR_INVALID_ARG;  // nothing to write
  if (!row_out && tgt_argmax) return SPEC_ERR_INVALID_ARG;  // the argmax comes from the row merge
  if (rows < 1 || vocab < 1) return SPEC_ERR_INVALID_ARG;
  if (!(temperature > 0.0f) || isinf(temperature) || !(draft_temperature > 0.0f) || isinf(draft_temperature))
    return SPEC_ERR_INVALID_ARG;
  if ((parent == nullptr) != (n_nodes == nullptr)) return SPEC_ERR_INVALID_ARG;  // the tree: both or neither
  if (parent && (row_out || n_max < 1 || n_max > 64 || rows % n_max)) return SPEC_ERR_INVALID_ARG;
  const size_t one = sm_set_bytes(rows, vocab);
  if (!workspace || workspace_bytes < 2 * one) return SPEC_ERR_WORKSPACE;
  SmSet A = make_set(tgt_logits, rows, temperature, tgt_max, tgt_sumexp, tgt_argmax);
  SmSet B = make_set(dft_logits, rows, draft_temperature, dft_max, dft_sumexp, nullptr);
  sm_set_carve((char*)workspace, rows, vocab, &A, tgt_chunk_max, tgt_chunk_sum);
  sm_set_carve((char*)workspace + one, rows, vocab, &B, dft_chunk_max, dft_chunk_sum);
  B.parent = parent;
  B.n_nodes = n_nodes;
  B.n_max = n_max;
  return launch_stats(A, B, vocab, status, (hipStream_t)stream, row_out, comb);
}
}  // namespace spectree

extern "C" int spec_tree_softmax_pair(const float* tgt_logits, float temperature, const float* dft_logits,
                                      float draft_temperature, int64_t rows, int32_t vocab, const int32_t* parent,
                                      const int32_t* n_nodes, int32_t n_max, float* tgt_max,
                                      float* tgt_sumexp, int32_t* tgt_argmax, float* tgt_chunk_max,
                                      double* tgt_chunk_sum, float* dft_max, float* dft_sumexp, float* dft_chunk_max,
                                      double* dft_chunk_sum, void* workspace, size_t workspace_bytes,
                                      int32_t* status, void* stream) {
  return spectree::softmax_pair_call(tgt_logits, temperature, dft_logits, draft_temperature, rows, vocab, parent,
                                     n_nodes, n_max, tgt_max, tgt_sumexp, tgt_argmax, tgt_chunk_max, tgt_chunk_sum,
                                     dft_max, dft_sumexp, dft_chunk_max, dft_chunk_sum, workspace, workspace_bytes,
                                     status, stream, nullptr);
}
