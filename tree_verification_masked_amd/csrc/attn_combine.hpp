// The tree attention's launch arguments and its split combine, shared by the
// attention call (which launches the combine itself) and the verification step's
// logit pass (which runs the combine's rows as extra workgroups of its own launch).
#pragma once

#include "common.hpp"

namespace spectree {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  int32_t page_size, kv_capacity, n_pages;
  const int32_t* ctx_len;
  const int32_t* n_nodes;
  const int32_t* parent;  // the tree's parent links (ancestor rows built in the launch), or
  const uint64_t* anc;    // the ancestor rows themselves: exactly one is given
  int32_t batch, n_max, hq, hkv, head_dim, max_kv_len;
  float scale_log2;  // scale * log2(e): scores live in the log2 domain
  int32_t S, split_len, qblocks;
  float* mpart;    // [S, B, n_max, hq]     split max (log2 domain)
  float* lpart;    // [S, B, n_max, hq]     split sum of exponentials
  void* opart;     // [S, B, n_max, hq, D]  split output divided by its sum (0 if the sum is 0),
                   // in the element type of Q/K/V (bf16 or fp32)
  int32_t* status;
  // MFMA path with one split: the split writes the output rows directly (no partials,
  // no combine launch)
  int32_t direct;
  void* out;       // [B, n_max, hq, D] (direct)
};

// Length of the logical KV of a request with n nodes after ctx prompt keys, or -1
// when the request cannot be served.
__device__ inline int request_len_of(const AttnArgs& a, int n, int ctx) {
  if (n < 1 || n > a.n_max || ctx < 0) return -1;
  const int64_t len = (int64_t)ctx + n;
  const int64_t cap = a.block_table ? (int64_t)a.kv_capacity * a.page_size : (int64_t)a.kv_capacity;
  if (len > a.max_kv_len || len > cap) return -1;
  return (int)len;
}
__device__ inline int request_len(const AttnArgs& a, int b) { return request_len_of(a, a.n_nodes[b], a.ctx_len[b]); }

// ---------------------------------------------------------------------------
// Split combine: one wave per output row (b, node, head)
// ---------------------------------------------------------------------------
// NV consecutive elements as one load.
template <typename T, int NV>
__device__ inline void load_elems(const T* p, float (&x)[NV]) {
  if constexpr (sizeof(T) == 2 && NV == 2) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    x[0] = __uint_as_float(u << 16);
    x[1] = __uint_as_float(u & 0xffff0000u);
  } else if constexpr (sizeof(T) == 4 && NV == 2) {
    const float2 f = *reinterpret_cast<const float2*>(p);
    x[0] = f.x;
    x[1] = f.y;
  } else {
#pragma unroll
    for (int v = 0; v < NV; ++v) x[v] = (float)p[v];
  }
}

// Output row `rowid` (b, node, head) from the split partials, by one whole wave;
// kBatch splits' partial outputs are loaded at once.
template <int D, typename T, int kBatch = 16>
__device__ inline void attn_combine_row(const AttnArgs& a, T* __restrict__ out, int64_t rowid) {
  constexpr int NV = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.batch * a.n_max * a.hq;
  if (rowid >= rows) return;
  const int node = (int)((rowid / a.hq) % a.n_max);
  const int b = (int)(rowid / ((int64_t)a.hq * a.n_max));
  const int64_t stride = rows;
  // Every load is issued before any result is used: the request's lengths, the
  // split maxima and sums (lane s holds split s) and the first kBatch partial
  // outputs (every row of every split is written by the attention launch, so these
  // addresses are valid whether or not the row turns out live).
  const int len = request_len(a, b);
  // (built from parent links, the ancestor rows of a request that is not a tree were
  // all dead in the attention launch, so their partial sums are zero)
  const uint64_t anc_row = a.anc ? a.anc[(int64_t)b * a.n_max + node] : (1ull << node);
  const int nb = a.n_nodes[b];
  const int sl = min(lane, a.S - 1);
  const float m_l = a.mpart[sl * stride + rowid], l_l = a.lpart[sl * stride + rowid];
  float vals[kBatch][NV];
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    load_elems<T, NV>((const T*)a.opart + (min(j, a.S - 1) * stride + rowid) * D + NV * lane, vals[j]);
  const bool live = len >= 0 && node < nb && ((anc_row >> node) & 1ull);
  if (len < 0 && node == 0 && rowid % a.hq == 0 && lane == 0) report(a.status, SPEC_ERR_BAD_INPUT);
  float res[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) res[v] = 0.0f;
  // split weights w_s = l_s 2^(m_s - m) (an empty split has m_s = -inf, l_s = 0);
  // lane s keeps w_s for s < 64, later splits (very long contexts) are reloaded
  float mx = lane < a.S ? m_l : -INFINITY;
  for (int s2 = lane + 64; s2 < a.S; s2 += 64) mx = fmaxf(mx, a.mpart[s2 * stride + rowid]);
  const float m = wave_max_f(mx);
  auto weight = [&](float ms, float ls) { return m > -INFINITY ? ls * __builtin_amdgcn_exp2f(ms - m) : 0.0f; };
  const float w_l = lane < a.S ? weight(m_l, l_l) : 0.0f;
  float lsum = w_l;
  for (int s2 = lane + 64; s2 < a.S; s2 += 64) lsum += weight(a.mpart[s2 * stride + rowid], a.lpart[s2 * stride + rowid]);
  const float L = wave_sum_f(lsum);
  auto w_of = [&](int s2) -> float {  // uniform s2
    if (s2 < 64) return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(w_l), s2));
    return weight(a.mpart[s2 * stride + rowid], a.lpart[s2 * stride + rowid]);
  };
  if (live && L > 0.0f) {  // wave-uniform
    float acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = 0.0f;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (j < a.S) {
        const float w = w_of(j);
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = fmaf(vals[j][v], w, acc[v]);
      }
    }
    for (int s0 = kBatch; s0 < a.S; s0 += kBatch) {  // more splits than one batch
      float more[kBatch][NV];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        load_elems<T, NV>((const T*)a.opart + (min(s0 + j, a.S - 1) * stride + rowid) * D + NV * lane, more[j]);
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (s0 + j < a.S) {
          const float w = w_of(s0 + j);
#pragma unroll
          for (int v = 0; v < NV; ++v) acc[v] = fmaf(more[j][v], w, acc[v]);
        }
      }
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int v = 0; v < NV; ++v) res[v] = acc[v] * inv;
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) out[rowid * D + NV * lane + v] = (T)res[v];
}

// A combine whose launch was handed to another kernel: `rows` output rows (0: none),
// in the element type and head size of the call.
struct AttnCombine {
  AttnArgs a;
  void* out;
  int32_t dtype, head_dim;
  int64_t rows;
};

}  // namespace spectree
