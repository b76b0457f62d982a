// Tree-masked split-KV GQA attention.
//
// Tree-verification notes (zhangshuibai.github.io), "Tree Verification 详解" part B:
// every flattened tree node attends to the prompt, its ancestors and itself, so its
// output equals an ordinary causal run of prompt + Path(root, node); part D.2: the
// node-to-prompt product is O(N * P) and dominates, the node-to-tree part is sparse.
// "EAGLE-4 Technical Deepdive" (blog.fal.ai), "EAGLE-4 verification trees and
// harness": the mask shows the shared prefix, the ancestors and the token itself.
//
// Work split: the logical key range [0, max_kv_len) is cut into S splits of whole
// 64-key tiles; a workgroup owns (request, KV head, query block, split) and keeps an
// online softmax per query row.  The rows of one KV head are its n_max * hq/hkv
// (node, query head) pairs, so K/V tiles are loaded once per workgroup and reused by
// every row (GQA).  Partials (max, sum, unnormalised output) go to the workspace and
// a combine kernel merges the splits with a log-sum-exp rescale.
//
//  * MFMA path (bf16, >= 16 rows per KV head): four waves of 32 rows each.  Scores
//    are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so each
//    lane ends up owning one query row; that accumulator layout is exactly the B
//    operand of O^T = V^T P^T for a fixed permutation of the 16 keys of a step, and
//    V is staged transposed in LDS in that key order.
//  * Shuffle path (fp32, or fewer than 16 rows): lane j of a wave scores key j of
//    the tile against one row, the row softmax uses wave reductions, and P V is
//    accumulated with one lane per head dimension.
#include <algorithm>

#include "common.hpp"

namespace spectree {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;           // keys per tile
constexpr int kMfmaRowsPerWg = 128; // 4 waves x 32 rows
constexpr int kShflRowsPerWg = 16;  // 4 waves x 4 rows
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  int32_t page_size, kv_capacity, n_pages;
  const int32_t* ctx_len;
  const int32_t* n_nodes;
  const uint64_t* anc;
  int32_t batch, n_max, hq, hkv, head_dim, max_kv_len;
  float scale_log2;  // scale * log2(e): scores live in the log2 domain
  int32_t S, split_len, qblocks;
  float* opart;  // [S, B, n_max, hq, D]
  float* mpart;  // [S, B, n_max, hq]
  float* lpart;  // [S, B, n_max, hq]
  int32_t* status;
};

// Length of request b's logical KV, or -1 when the request cannot be served.
__device__ inline int request_len(const AttnArgs& a, int b) {
  const int n = a.n_nodes[b], ctx = a.ctx_len[b];
  if (n < 1 || n > a.n_max || ctx < 0) return -1;
  const int64_t len = (int64_t)ctx + n;
  const int64_t cap = a.block_table ? (int64_t)a.kv_capacity * a.page_size : (int64_t)a.kv_capacity;
  if (len > a.max_kv_len || len > cap) return -1;
  return (int)len;
}

// Element offset of key t (< len) of request b, KV head g; -1 for a bad page id.
__device__ inline int64_t kv_off(const AttnArgs& a, int b, int t, int g) {
  if (!a.block_table) return (((int64_t)b * a.kv_capacity + t) * a.hkv + g) * a.head_dim;
  const int page = a.block_table[(int64_t)b * a.kv_capacity + t / a.page_size];
  if (page < 0 || page >= a.n_pages) return -1;
  return (((int64_t)page * a.page_size + t % a.page_size) * a.hkv + g) * a.head_dim;
}

__device__ inline bool key_visible(int t, int len, int ctx, uint64_t anc_row) {
  if (t >= len) return false;
  if (t < ctx) return true;
  return (anc_row >> (t - ctx)) & 1ull;
}

// ---------------------------------------------------------------------------
// MFMA path
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnArgs a) {
  constexpr int KS = D + 8;      // LDS row stride (bf16) of the K tile
  constexpr int VS = kTile + 8;  // LDS row stride (bf16) of the transposed V tile
  constexpr int PIECES = kTile * D / 8;  // 16-byte pieces per tile
  constexpr int PER_THREAD = PIECES / 256;
  __shared__ __attribute__((aligned(16))) __bf16 sK[kTile * KS];
  __shared__ __attribute__((aligned(16))) __bf16 sVt[D * VS];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int blk = blockIdx.x;
  const int s = blk % a.S;
  blk /= a.S;
  const int qb = blk % a.qblocks;
  blk /= a.qblocks;
  const int g = blk % a.hkv;
  const int b = blk / a.hkv;
  const int hpg = a.hq / a.hkv;
  const int G = a.n_max * hpg;

  const int len = request_len(a, b);
  const int n = a.n_nodes[b];
  const int ctx = a.ctx_len[b];
  // this lane's query row
  const int r = qb * kMfmaRowsPerWg + wid * 32 + (lane & 31);
  const int node = r / hpg;
  const int h = g * hpg + r % hpg;
  const bool row_live = len >= 0 && r < G && node < n;
  const uint64_t anc_row = row_live ? a.anc[(int64_t)b * a.n_max + node] : 0ull;

  const int k_begin = s * a.split_len;
  const int k_end = min(k_begin + a.split_len, len < 0 ? 0 : len);

  // Q fragments: lane holds row r, dims kk*16 + 8*(lane/32) .. +8
  bf16x8 qf[D / 16];
  {
    const __bf16* qrow = (const __bf16*)a.q + (((int64_t)b * a.n_max + node) * a.hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (row_live && anc_row)
        qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + kk * 16 + 8 * (lane >> 5));
      else
        qf[kk] = bf16x8{};
    }
  }
  f32x16 acc_o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc_o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  const __bf16* kbase = (const __bf16*)a.k;
  const __bf16* vbase = (const __bf16*)a.v;
  uint4 kreg[PER_THREAD], vreg[PER_THREAD];
  int bad_page = 0;
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int p = tid + j * 256;
      const int key = p / (D / 8), dc = p % (D / 8);
      const int t = t0 + key;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (t < k_end) {
        const int64_t off = kv_off(a, b, t, g);
        if (off >= 0) {
          kv = *reinterpret_cast<const uint4*>(kbase + off + dc * 8);
          vv = *reinterpret_cast<const uint4*>(vbase + off + dc * 8);
        } else {
          bad_page = 1;
        }
      }
      kreg[j] = kv;
      vreg[j] = vv;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int p = tid + j * 256;
      const int key = p / (D / 8), dc = p % (D / 8);
      *reinterpret_cast<uint4*>(&sK[key * KS + dc * 8]) = kreg[j];
      const __bf16* vv = reinterpret_cast<const __bf16*>(&vreg[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) sVt[(dc * 8 + e) * VS + key] = vv[e];
    }
  };

  const int n_tiles = k_end > k_begin ? (k_end - k_begin + kTile - 1) / kTile : 0;
  if (n_tiles > 0) load_tile(k_begin);
  for (int it = 0; it < n_tiles; ++it) {
    const int t0 = k_begin + it * kTile;
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (it + 1 < n_tiles) load_tile(t0 + kTile);  // overlaps the math below

    // ---- S^T = K Q^T for two 32-key blocks ----
    f32x16 acc_s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      acc_s[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(&sK[(kb * 32 + (lane & 31)) * KS + kk * 16 + 8 * (lane >> 5)]);
        acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], acc_s[kb], 0, 0, 0);
      }
    }
    // ---- mask, scale, online softmax (lane owns row lane%32; lane^32 holds the other keys) ----
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kb * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int t = t0 + key;
        const bool vis = row_live && t < k_end && key_visible(t, len, ctx, anc_row);
        const float sc = vis ? acc_s[kb][e] * a.scale_log2 : -INFINITY;
        acc_s[kb][e] = sc;
        tmax = fmaxf(tmax, sc);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.0f;
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = (m_new == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(acc_s[kb][e] - m_new);
        psum += p;
        pf[kb * 2 + (e >> 3)][e & 7] = (__bf16)p;
      }
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc_o[db] *= alpha;
    // ---- O^T += V^T P^T; k-step ks covers keys 16*ks .. 16*ks+15 in the permuted order ----
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const __bf16* vrow = &sVt[(db * 32 + (lane & 31)) * VS + 4 * (lane >> 5)];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow + ks * 16);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + ks * 16 + 8);
        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], acc_o[db], 0, 0, 0);
      }
    }
  }
  if (bad_page) report(a.status, SPEC_ERR_BAD_INPUT);
  // ---- write this split's partials for the lane's row ----
  if (r < G && node < a.n_max) {
    const int64_t prow = (((int64_t)s * a.batch + b) * a.n_max + node) * a.hq + h;
    if (lane < 32) {
      a.mpart[prow] = m_run;
      a.lpart[prow] = l_run;
    }
    float* orow = a.opart + prow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = db * 32 + 8 * e4 + 4 * (lane >> 5);
        *reinterpret_cast<float4*>(orow + d) =
            make_float4(acc_o[db][4 * e4 + 0], acc_o[db][4 * e4 + 1], acc_o[db][4 * e4 + 2], acc_o[db][4 * e4 + 3]);
      }
  }
}

// ---------------------------------------------------------------------------
// Shuffle path
// ---------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(256) void attn_shfl_kernel(AttnArgs a) {
  constexpr int NV = D / 64;  // head dims per lane
  __shared__ float sQ[kShflRowsPerWg * D];
  __shared__ float sK[kTile * (D + 1)];
  __shared__ float sV[kTile * D];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int blk = blockIdx.x;
  const int s = blk % a.S;
  blk /= a.S;
  const int qb = blk % a.qblocks;
  blk /= a.qblocks;
  const int g = blk % a.hkv;
  const int b = blk / a.hkv;
  const int hpg = a.hq / a.hkv;
  const int G = a.n_max * hpg;
  const int len = request_len(a, b);
  const int n = a.n_nodes[b];
  const int ctx = a.ctx_len[b];
  const int k_begin = s * a.split_len;
  const int k_end = min(k_begin + a.split_len, len < 0 ? 0 : len);
  const T* qg = (const T*)a.q;
  const T* kg = (const T*)a.k;
  const T* vg = (const T*)a.v;

  for (int x = tid; x < kShflRowsPerWg * D; x += 256) {
    const int rr = qb * kShflRowsPerWg + x / D;
    const int node = rr / hpg, h = g * hpg + rr % hpg;
    float val = 0.0f;
    if (rr < G && node < n && len >= 0) val = (float)qg[(((int64_t)b * a.n_max + node) * a.hq + h) * D + x % D];
    sQ[x] = val;
  }
  // per-wave rows: wid, wid + 4, wid + 8, wid + 12
  float m_run[4], l_run[4], o[4][NV];
  uint64_t anc_row[4];
  bool live[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = qb * kShflRowsPerWg + wid + 4 * j;
    const int node = rr / hpg;
    live[j] = len >= 0 && rr < G && node < n;
    anc_row[j] = live[j] ? a.anc[(int64_t)b * a.n_max + node] : 0ull;
    m_run[j] = -INFINITY;
    l_run[j] = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) o[j][v] = 0.0f;
  }
  int bad_page = 0;
  for (int t0 = k_begin; t0 < k_end; t0 += kTile) {
    __syncthreads();
    for (int x = tid; x < kTile * D; x += 256) {
      const int key = x / D, d = x % D, t = t0 + key;
      float kv = 0.0f, vv = 0.0f;
      if (t < k_end) {
        const int64_t off = kv_off(a, b, t, g);
        if (off >= 0) {
          kv = (float)kg[off + d];
          vv = (float)vg[off + d];
        } else {
          bad_page = 1;
        }
      }
      sK[key * (D + 1) + d] = kv;
      sV[key * D + d] = vv;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!live[j]) continue;  // uniform per wave
      const int rl = wid + 4 * j;
      const int t = t0 + lane;
      float sc = 0.0f;
      for (int d = 0; d < D; ++d) sc = fmaf(sQ[rl * D + d], sK[lane * (D + 1) + d], sc);
      const bool vis = t < k_end && key_visible(t, len, ctx, anc_row[j]);
      sc = vis ? sc * a.scale_log2 : -INFINITY;
      const float tmax = wave_max_f(sc);
      const float m_new = fmaxf(m_run[j], tmax);
      if (m_new == -INFINITY) continue;
      const float alpha = __builtin_amdgcn_exp2f(m_run[j] - m_new);
      const float p = __builtin_amdgcn_exp2f(sc - m_new);
      l_run[j] = l_run[j] * alpha + wave_sum_f(p);
      m_run[j] = m_new;
#pragma unroll
      for (int v = 0; v < NV; ++v) o[j][v] *= alpha;
      for (int key = 0; key < kTile; ++key) {
        const float pk = __shfl(p, key);
#pragma unroll
        for (int v = 0; v < NV; ++v) o[j][v] = fmaf(pk, sV[key * D + lane + 64 * v], o[j][v]);
      }
    }
  }
  if (bad_page) report(a.status, SPEC_ERR_BAD_INPUT);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = qb * kShflRowsPerWg + wid + 4 * j;
    if (rr >= G) continue;
    const int node = rr / hpg, h = g * hpg + rr % hpg;
    const int64_t prow = (((int64_t)s * a.batch + b) * a.n_max + node) * a.hq + h;
    if (lane == 0) {
      a.mpart[prow] = m_run[j];
      a.lpart[prow] = l_run[j];
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) a.opart[prow * D + lane + 64 * v] = o[j][v];
  }
}

// ---------------------------------------------------------------------------
// Split combine: one wave per output row (b, node, head)
// ---------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, T* __restrict__ out) {
  constexpr int NV = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t rowid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)a.batch * a.n_max * a.hq;
  if (rowid >= rows) return;
  const int h = (int)(rowid % a.hq);
  const int node = (int)((rowid / a.hq) % a.n_max);
  const int b = (int)(rowid / ((int64_t)a.hq * a.n_max));
  const int len = request_len(a, b);
  const uint64_t anc_row = a.anc[(int64_t)b * a.n_max + node];
  const bool live = len >= 0 && node < a.n_nodes[b] && ((anc_row >> node) & 1ull);
  if (len < 0 && node == 0 && h == 0 && lane == 0) report(a.status, SPEC_ERR_BAD_INPUT);
  float res[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) res[v] = 0.0f;
  if (live) {
    const int64_t stride = (int64_t)a.batch * a.n_max * a.hq;
    float m = -INFINITY;
    for (int s = 0; s < a.S; ++s) m = fmaxf(m, a.mpart[s * stride + rowid]);
    if (m > -INFINITY) {
      float L = 0.0f;
      float acc[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] = 0.0f;
      for (int s = 0; s < a.S; ++s) {
        const float ms = a.mpart[s * stride + rowid];
        if (ms == -INFINITY) continue;
        const float w = __builtin_amdgcn_exp2f(ms - m);
        L = fmaf(a.lpart[s * stride + rowid], w, L);
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = fmaf(a.opart[(s * stride + rowid) * D + lane + 64 * v], w, acc[v]);
      }
      const float inv = 1.0f / L;
#pragma unroll
      for (int v = 0; v < NV; ++v) res[v] = acc[v] * inv;
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) out[rowid * D + lane + 64 * v] = (T)res[v];
}

struct AttnPlan {
  bool mfma;
  int S, split_len, qblocks;
};

inline AttnPlan make_plan(int32_t batch, int32_t n_max, int32_t hq, int32_t hkv, int32_t max_kv_len, int32_t dtype) {
  AttnPlan p;
  const int G = n_max * (hq / hkv);
  p.mfma = dtype == SPEC_BF16 && G >= 16;
  const int rows_per_wg = p.mfma ? kMfmaRowsPerWg : kShflRowsPerWg;
  p.qblocks = (G + rows_per_wg - 1) / rows_per_wg;
  const int tiles = max(1, (max_kv_len + kTile - 1) / kTile);
  const int64_t base = (int64_t)batch * hkv * p.qblocks;
  const int64_t target = 512;  // two workgroups per CU
  int S = (int)std::min<int64_t>((target + base - 1) / base, tiles);
  S = std::max(S, 1);
  const int tiles_per_split = (tiles + S - 1) / S;
  p.S = (tiles + tiles_per_split - 1) / tiles_per_split;
  p.split_len = tiles_per_split * kTile;
  return p;
}

inline size_t attn_ws_bytes(const AttnPlan& p, int32_t batch, int32_t n_max, int32_t hq, int32_t D) {
  const size_t rows = (size_t)p.S * batch * n_max * hq;
  return rows * D * sizeof(float) + 2 * rows * sizeof(float);
}

}  // namespace spectree

extern "C" size_t spec_tree_attention_workspace_size(int32_t batch, int32_t n_max, int32_t hq, int32_t hkv,
                                                     int32_t head_dim, int32_t max_kv_len) {
  using namespace spectree;
  if (batch < 1 || n_max < 1 || hq < 1 || hkv < 1 || hq % hkv || head_dim < 1 || max_kv_len < 1) return 0;
  // the MFMA plan has fewer splits; size for the larger of the two
  const AttnPlan p0 = make_plan(batch, n_max, hq, hkv, max_kv_len, SPEC_F32);
  const AttnPlan p1 = make_plan(batch, n_max, hq, hkv, max_kv_len, SPEC_BF16);
  return std::max(attn_ws_bytes(p0, batch, n_max, hq, head_dim), attn_ws_bytes(p1, batch, n_max, hq, head_dim));
}

extern "C" int spec_tree_attention(const void* q, const void* k, const void* v, int32_t dtype,
                                   const int32_t* block_table, int32_t page_size, int32_t kv_capacity,
                                   int32_t n_pages, const int32_t* ctx_len, const int32_t* n_nodes,
                                   const uint64_t* anc_mask, int32_t batch, int32_t n_max, int32_t hq, int32_t hkv,
                                   int32_t head_dim, int32_t max_kv_len, float scale, void* out, void* workspace,
                                   size_t workspace_bytes, int32_t* status, void* stream) {
  using namespace spectree;
  if (!q || !k || !v || !ctx_len || !n_nodes || !anc_mask || !out) return SPEC_ERR_INVALID_ARG;
  if (batch < 1 || n_max < 1 || n_max > 64 || hq < 1 || hkv < 1 || hq % hkv != 0) return SPEC_ERR_INVALID_ARG;
  if (kv_capacity < 1 || max_kv_len < 1 || !(scale > 0.0f) || isinf(scale)) return SPEC_ERR_INVALID_ARG;
  if (block_table && (page_size < 1 || n_pages < 1)) return SPEC_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return SPEC_ERR_UNSUPPORTED;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_UNSUPPORTED;
  const AttnPlan p = make_plan(batch, n_max, hq, hkv, max_kv_len, dtype);
  if (!workspace || workspace_bytes < attn_ws_bytes(p, batch, n_max, hq, head_dim)) return SPEC_ERR_WORKSPACE;
  const int64_t grid = (int64_t)batch * hkv * p.qblocks * p.S;
  if (grid > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.block_table = block_table;
  a.page_size = page_size;
  a.kv_capacity = kv_capacity;
  a.n_pages = n_pages;
  a.ctx_len = ctx_len;
  a.n_nodes = n_nodes;
  a.anc = anc_mask;
  a.batch = batch;
  a.n_max = n_max;
  a.hq = hq;
  a.hkv = hkv;
  a.head_dim = head_dim;
  a.max_kv_len = max_kv_len;
  a.scale_log2 = scale * kLog2e;
  a.S = p.S;
  a.split_len = p.split_len;
  a.qblocks = p.qblocks;
  const size_t rows = (size_t)p.S * batch * n_max * hq;
  a.opart = (float*)workspace;
  a.mpart = a.opart + rows * head_dim;
  a.lpart = a.mpart + rows;
  a.status = status;
  hipStream_t st = (hipStream_t)stream;
  const dim3 g1((unsigned)grid), blk(256);
  if (p.mfma) {
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_mfma_kernel<128>, g1, blk, 0, st, a);
    else
      hipLaunchKernelGGL(attn_mfma_kernel<64>, g1, blk, 0, st, a);
  } else if (dtype == SPEC_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_shfl_kernel<128, __bf16>), g1, blk, 0, st, a);
    else
      hipLaunchKernelGGL((attn_shfl_kernel<64, __bf16>), g1, blk, 0, st, a);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_shfl_kernel<128, float>), g1, blk, 0, st, a);
    else
      hipLaunchKernelGGL((attn_shfl_kernel<64, float>), g1, blk, 0, st, a);
  }
  SPEC_LAUNCH_CHECK();
  const int64_t out_rows = (int64_t)batch * n_max * hq;
  const dim3 g2((unsigned)((out_rows + 3) / 4));
  if (dtype == SPEC_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_combine_kernel<128, __bf16>), g2, blk, 0, st, a, (__bf16*)out);
    else
      hipLaunchKernelGGL((attn_combine_kernel<64, __bf16>), g2, blk, 0, st, a, (__bf16*)out);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_combine_kernel<128, float>), g2, blk, 0, st, a, (float*)out);
    else
      hipLaunchKernelGGL((attn_combine_kernel<64, float>), g2, blk, 0, st, a, (float*)out);
  }
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}
