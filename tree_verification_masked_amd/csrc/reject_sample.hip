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
// Residual in closed form.  With a fixed q, after j rejections the residual is
//   r_j = max(0, p - c_j q) / W(c_j),   W(c) = sum_x max(0, p(x) - c q(x)),
// c_0 = 0, W(0) = 1 and c_{j+1} = c_j + W(c_j) (kept at c_j when W(c_{j+1}) = 0,
// where the residual is left unchanged).  So a sibling test needs only p(x), q(x)
// of one token plus the scalars (c_j, W(c_j)), and each further sibling costs one
// reduction pass over the vocabulary instead of a rewritten residual vector.
//
// Work layout: one workgroup per request walks the tree lazily from the root (only
// nodes on the committed path are evaluated; uniforms are indexed by node, so the
// result equals evaluating every node).  Vocabulary passes are spread over the
// workgroup with coalesced loads; every reduction has a fixed order, so results
// are bitwise reproducible.  Tested tokens use fp64 exp; pass elements use the
// fp32 exp2 of the softmax kernel with fp64 accumulation.
#include "common.hpp"

namespace spectree {

constexpr int kRjMaxWaves = 16;

struct RowView {
  const float* lt;   // target logits of the node
  const float* ld;   // draft logits of the node
  float mt, md;      // row maxima
  double izt, izd;   // 1 / row sums of exp
  ExpScale est, esd; // exp scales for 1/T and 1/T_d
};

// w(x) = max(0, p(x) - c q(x)); c == 0 is p itself (draft row not read).
__device__ inline double resid_elem(const RowView& r, int t, double c) {
  const double p = (double)exp_scaled(r.lt[t] - r.mt, r.est) * r.izt;
  if (c == 0.0) return p;
  const double q = (double)exp_scaled(r.ld[t] - r.md, r.esd) * r.izd;
  return fmax(0.0, p - c * q);
}

// W(c) over the vocabulary, identical in every thread of the block.
__device__ double block_W(const RowView& r, int vocab, double c, double* s_red) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw = blockDim.x >> 6;
  double acc = 0.0;
  for (int t = tid; t < vocab; t += blockDim.x) acc += resid_elem(r, t, c);
  acc = wave_sum_d(acc);
  __syncthreads();
  if (lane == 0) s_red[wid] = acc;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < nw; ++w) tot += s_red[w];
  return tot;
}

// Inverse-CDF draw from w(x) = max(0, p - c q) with uniform u: the smallest token
// whose running sum (ascending token order) exceeds u * S.  Wave w owns a
// contiguous token segment read 64 tokens at a time; sub-block sums come from an
// in-wave inclusive scan, and the segment totals are added in order, so the
// search pass below reproduces exactly the sums that located the crossing.
// Returns -1 when the total mass is zero.
__device__ int block_draw(const RowView& r, int vocab, double c, double u, double* s_red, int* s_int,
                          double& total) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw = blockDim.x >> 6;
  const int seg = ((vocab + nw * 64 - 1) / (nw * 64)) * 64;
  const int w0 = wid * seg, w1 = min(vocab, w0 + seg);
  double run = 0.0;
  int lastpos = -1;
  for (int base = w0; base < w1; base += 64) {
    const int t = base + lane;
    double val = 0.0;
    if (t < w1) {
      val = resid_elem(r, t, c);
      if (val > 0.0) lastpos = t;
    }
    const double incl = wave_incl_scan_d(val, lane);
    run += __shfl(incl, 63);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lastpos = max(lastpos, __shfl_xor(lastpos, o));
  __syncthreads();
  if (lane == 0) {
    s_red[wid] = run;
    s_int[wid] = lastpos;
  }
  __syncthreads();
  double S = 0.0;
  for (int w = 0; w < nw; ++w) S += s_red[w];
  const double target = u * S;
  double pre = 0.0;
  int ws = -1;
  for (int w = 0; w < nw; ++w) {
    if (pre + s_red[w] > target) {
      ws = w;
      break;
    }
    pre += s_red[w];
  }
  int k = -1;
  if (ws < 0) {  // rounding left no crossing: largest token with positive mass
    for (int w = 0; w < nw; ++w) k = max(k, s_int[w]);
  } else if (wid == ws) {
    double rr = 0.0;
    int found = -1;
    for (int base = w0; base < w1; base += 64) {
      const int t = base + lane;
      const double val = (t < w1) ? resid_elem(r, t, c) : 0.0;
      const double incl = wave_incl_scan_d(val, lane);
      const double tot = __shfl(incl, 63);
      if (pre + (rr + tot) > target) {
        const uint64_t hit = __ballot(pre + (rr + incl) > target);
        found = base + (int)__builtin_ctzll(hit);
        break;
      }
      rr += tot;
    }
    if (found < 0) found = s_int[ws];
    if (lane == 0) s_int[kRjMaxWaves] = found;
  }
  __syncthreads();
  if (ws >= 0) k = s_int[kRjMaxWaves];
  total = S;
  __syncthreads();
  return k;
}

__global__ __launch_bounds__(1024) void reject_sample_kernel(
    const float* __restrict__ tgt_logits, const float* __restrict__ tgt_max, const float* __restrict__ tgt_sumexp,
    const int32_t* __restrict__ tgt_argmax, double inv_t, ExpScale est, const float* __restrict__ dft_logits,
    const float* __restrict__ dft_max, const float* __restrict__ dft_sumexp, double inv_td, ExpScale esd,
    int greedy, const int32_t* __restrict__ tokens, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ n_nodes, const float* __restrict__ u_accept, const float* __restrict__ u_sample,
    int32_t n_max, int32_t vocab, int32_t* __restrict__ accepted_child, int32_t* __restrict__ term_token,
    int32_t* status) {
  __shared__ int s_par[64];
  __shared__ int s_tok[64];
  __shared__ double s_red[kRjMaxWaves];
  __shared__ int s_int[kRjMaxWaves + 1];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int64_t base = (int64_t)b * n_max;
  const int n = n_nodes[b];
  if (tid < n_max) {
    accepted_child[base + tid] = SPEC_NODE_NOT_EVALUATED;
    term_token[base + tid] = SPEC_NODE_NOT_EVALUATED;
  }
  const bool n_ok = n >= 1 && n <= n_max;
  if (tid < 64) {
    s_par[tid] = (n_ok && tid < n) ? parent[base + tid] : -1;
    s_tok[tid] = (n_ok && tid < n) ? tokens[base + tid] : 0;
  }
  __syncthreads();
  // request validation: tree links and token ids (every thread reaches the same verdict)
  int verdict = n_ok ? 0 : SPEC_ERR_BAD_TREE;
  if (n_ok) {
    if (s_par[0] != -1) verdict = SPEC_ERR_BAD_TREE;
    for (int i = 1; i < n && verdict == 0; ++i)
      if (s_par[i] < 0 || s_par[i] >= i) verdict = SPEC_ERR_BAD_TREE;
    for (int i = 1; i < n && verdict == 0; ++i)
      if (s_tok[i] < 0 || s_tok[i] >= vocab) verdict = SPEC_ERR_BAD_INPUT;
  }
  int cur = 0;
  for (int step = 0; verdict == 0 && step < n; ++step) {
    const int64_t row = base + cur;
    RowView rv;
    rv.lt = tgt_logits + row * (int64_t)vocab;
    rv.mt = tgt_max[row];
    if (isnan(rv.mt)) {
      verdict = SPEC_ERR_BAD_INPUT;
      break;
    }
    if (greedy) {
      const int a = tgt_argmax[row];
      int acc = SPEC_NODE_NONE;
      for (int c = cur + 1; c < n; ++c)
        if (s_par[c] == cur && s_tok[c] == a) {
          acc = c;
          break;
        }
      if (tid == 0) accepted_child[row] = acc;
      if (acc >= 0) {
        cur = acc;
        continue;
      }
      if (tid == 0) term_token[row] = a;
      break;
    }
    rv.ld = dft_logits + row * (int64_t)vocab;
    rv.md = dft_max[row];
    if (isnan(rv.md)) {
      verdict = SPEC_ERR_BAD_INPUT;
      break;
    }
    rv.izt = 1.0 / (double)tgt_sumexp[row];
    rv.izd = 1.0 / (double)dft_sumexp[row];
    rv.est = est;
    rv.esd = esd;
    double cth = 0.0, W = 1.0;  // residual threshold and its mass W(cth)
    double c_prev = 0.0;
    bool pending = false;         // cth holds a last step whose mass is not yet known
    int acc = SPEC_NODE_NONE;
    for (int c = cur + 1; c < n; ++c) {
      if (s_par[c] != cur) continue;
      const int x = s_tok[c];
      const double px = exp(((double)rv.lt[x] - (double)rv.mt) * inv_t) * rv.izt;
      const double qx = exp(((double)rv.ld[x] - (double)rv.md) * inv_td) * rv.izd;
      const double num = fmax(0.0, px - cth * qx);
      const double ratio = qx > 0.0 ? num / (W * qx) : (num > 0.0 ? INFINITY : 0.0);
      if ((double)u_accept[base + c] < ratio) {
        acc = c;
        break;
      }
      // rejected.  The next residual's mass is needed now only if another sibling
      // follows; otherwise the draw pass below computes it.
      bool more = false;
      for (int c2 = c + 1; c2 < n; ++c2)
        if (s_par[c2] == cur) {
          more = true;
          break;
        }
      if (more) {
        const double cn = cth + W;
        const double Wn = block_W(rv, vocab, cn, s_red);
        if (Wn > 0.0) {
          cth = cn;
          W = Wn;
        }
      } else {
        c_prev = cth;
        cth = cth + W;
        pending = true;
      }
    }
    if (tid == 0) accepted_child[row] = acc;
    if (acc >= 0) {
      cur = acc;
      continue;
    }
    const double u = (double)u_sample[base + cur];
    double S = 0.0;
    int k = block_draw(rv, vocab, cth, u, s_red, s_int, S);
    if (pending && !(S > 0.0)) {  // zero-mass last step: the residual stays as it was
      k = block_draw(rv, vocab, c_prev, u, s_red, s_int, S);
    }
    if (tid == 0) term_token[row] = k;
    if (k < 0 && tid == 0) report(status, SPEC_ERR_BAD_INPUT);
    break;
  }
  __syncthreads();
  if (verdict != 0) {
    if (tid < n_max) {
      accepted_child[base + tid] = tid == 0 ? SPEC_NODE_BAD_REQUEST : SPEC_NODE_NOT_EVALUATED;
      term_token[base + tid] = SPEC_NODE_NOT_EVALUATED;
    }
    if (tid == 0) report(status, verdict);
  }
}

}  // namespace spectree

extern "C" size_t spec_tree_reject_sample_workspace_size(int32_t batch, int32_t n_max, int32_t vocab) {
  (void)batch;
  (void)n_max;
  (void)vocab;
  return 0;
}

extern "C" int spec_tree_reject_sample(const float* tgt_logits, const float* tgt_max, const float* tgt_sumexp,
                                       const int32_t* tgt_argmax, float temperature, const float* dft_logits,
                                       const float* dft_max, const float* dft_sumexp, float draft_temperature,
                                       const int32_t* tokens, const int32_t* parent, const int32_t* n_nodes,
                                       const float* u_accept, const float* u_sample, int32_t batch, int32_t n_max,
                                       int32_t vocab, int32_t* accepted_child, int32_t* term_token, void* workspace,
                                       size_t workspace_bytes, int32_t* status, void* stream) {
  using namespace spectree;
  (void)workspace;
  (void)workspace_bytes;
  if (!(temperature >= 0.0f) || isinf(temperature)) return SPEC_ERR_INVALID_ARG;
  const bool greedy = temperature == 0.0f;
  if (!tgt_logits || !tgt_max || !tokens || !parent || !n_nodes || !accepted_child || !term_token)
    return SPEC_ERR_INVALID_ARG;
  if (greedy && !tgt_argmax) return SPEC_ERR_INVALID_ARG;
  if (!greedy) {
    if (!tgt_sumexp || !dft_logits || !dft_max || !dft_sumexp || !u_accept || !u_sample) return SPEC_ERR_INVALID_ARG;
    if (!(draft_temperature > 0.0f) || isinf(draft_temperature)) return SPEC_ERR_INVALID_ARG;
  }
  if (batch < 1 || n_max < 1 || n_max > 64 || vocab < 1) return SPEC_ERR_INVALID_ARG;
  const double inv_t = greedy ? 0.0 : 1.0 / (double)temperature;
  const double inv_td = greedy ? 0.0 : 1.0 / (double)draft_temperature;
  // one wavefront is enough for small vocabularies; 16 for large rows
  const int threads = vocab <= 4096 ? 64 : 1024;
  hipLaunchKernelGGL(reject_sample_kernel, dim3((unsigned)batch), dim3(threads), 0, (hipStream_t)stream, tgt_logits,
                     tgt_max, tgt_sumexp, tgt_argmax, inv_t, make_exp_scale(inv_t), dft_logits, dft_max, dft_sumexp,
                     inv_td, make_exp_scale(inv_td), greedy ? 1 : 0, tokens, parent, n_nodes, u_accept, u_sample,
                     n_max, vocab, accepted_child, term_token, status);
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}
