// Per-node vocabulary softmax statistics.
//
// "The EAGLE Family" (consciousengines.com), "Why predict features instead of
// tokens?": the next-token distribution is the softmax of the LM-head output.
// Tree-verification notes, parts A and D.2: one softmax per tree node, N x |V|
// elements per verify, bound by memory bandwidth.
//
// One pass over the logits.  A row is cut into chunks of kChunk elements; each
// workgroup reads one chunk with 16-byte loads (every element read once), keeps it
// in registers, and produces the chunk's maximum, first argmax and
// sum exp((l - m_chunk) / T) accumulated in fp64.  The last workgroup to finish a
// row (device-scope counter in the workspace, reset by that workgroup) merges the
// chunk partials in chunk order: m = max m_c, Z = sum_c s_c exp((m_c - m) / T).
#include "common.hpp"

namespace spectree {

constexpr int kSmThreads = 256;
constexpr int kSmPerThread = 32;                      // fp32 elements held per thread
constexpr int kChunk = kSmThreads * kSmPerThread;     // 8192 elements per workgroup

struct SmWorkspace {
  float* cmax;     // [rows, nch]
  double* csum;    // [rows, nch]
  int32_t* carg;   // [rows, nch]
  int32_t* cbad;   // [rows, nch]
  uint32_t* count; // [rows]
};

inline int sm_chunks(int32_t vocab) { return (vocab + kChunk - 1) / kChunk; }

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline size_t sm_layout(int64_t rows, int32_t vocab, char* base, SmWorkspace* w) {
  const size_t n = (size_t)rows * (size_t)sm_chunks(vocab);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  char* p0 = take(n * sizeof(float));
  char* p1 = take(n * sizeof(double));
  char* p2 = take(n * sizeof(int32_t));
  char* p3 = take(n * sizeof(int32_t));
  char* p4 = take((size_t)rows * sizeof(uint32_t));
  if (w) {
    w->cmax = (float*)p0;
    w->csum = (double*)p1;
    w->carg = (int32_t*)p2;
    w->cbad = (int32_t*)p3;
    w->count = (uint32_t*)p4;
  }
  return off;
}

template <bool kVec>
__global__ __launch_bounds__(kSmThreads) void softmax_stats_kernel(const float* __restrict__ logits, int32_t vocab,
                                                                   int nch, double inv_t, ExpScale es, int greedy,
                                                                   SmWorkspace ws, float* __restrict__ row_max,
                                                                   float* __restrict__ row_sumexp,
                                                                   int32_t* __restrict__ row_argmax, int32_t* status) {
  const int chunk = (int)(blockIdx.x % (unsigned)nch);
  const int64_t row = (int64_t)(blockIdx.x / (unsigned)nch);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const float* src = logits + row * (int64_t)vocab;
  const int c0 = chunk * kChunk;

  // Element (k, v) of a thread is token c0 + (k * kSmThreads + tid) * 4 + v, so
  // consecutive threads read consecutive 16-byte pieces.
  float x[kSmPerThread];
#pragma unroll
  for (int k = 0; k < kSmPerThread / 4; ++k) {
    const int t = c0 + (k * kSmThreads + tid) * 4;
    if (kVec && t + 3 < vocab) {
      const float4 f = *reinterpret_cast<const float4*>(src + t);
      x[4 * k + 0] = f.x;
      x[4 * k + 1] = f.y;
      x[4 * k + 2] = f.z;
      x[4 * k + 3] = f.w;
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) x[4 * k + v] = (t + v < vocab) ? src[t + v] : -INFINITY;
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
      const int t = c0 + (k * kSmThreads + tid) * 4 + v;
      bad |= is_bad_logit(e) ? 1 : 0;
      if (e > m) {  // tokens are visited in increasing order per thread
        m = e;
        am = t;
      }
    }
  // block max / first argmax / bad flag
  __shared__ float s_m[kSmThreads / 64];
  __shared__ int s_a[kSmThreads / 64];
  __shared__ int s_b[kSmThreads / 64];
  __shared__ double s_s[kSmThreads / 64];
  {
    float wm = m;
    int wa = am;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float om = __shfl_xor(wm, o);
      const int oa = __shfl_xor(wa, o);
      if (om > wm || (om == wm && oa < wa)) {
        wm = om;
        wa = oa;
      }
    }
    const int wb = wave_or_i(bad);
    if (lane == 0) {
      s_m[wid] = wm;
      s_a[wid] = wa;
      s_b[wid] = wb;
    }
  }
  __syncthreads();
  float cm = s_m[0];
  int ca = s_a[0];
  int cb = s_b[0];
#pragma unroll
  for (int w = 1; w < kSmThreads / 64; ++w) {
    if (s_m[w] > cm || (s_m[w] == cm && s_a[w] < ca)) {
      cm = s_m[w];
      ca = s_a[w];
    }
    cb |= s_b[w];
  }
  double csum = 0.0;
  if (!greedy && cm > -INFINITY) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kSmPerThread; ++k) acc += (double)exp_scaled(x[k] - cm, es);
    acc = wave_sum_d(acc);
    if (lane == 0) s_s[wid] = acc;
    __syncthreads();
    csum = s_s[0];
#pragma unroll
    for (int w = 1; w < kSmThreads / 64; ++w) csum += s_s[w];
  }
  const int64_t slot = row * nch + chunk;
  __shared__ int s_last;
  if (tid == 0) {
    ws.cmax[slot] = cm;
    ws.csum[slot] = csum;
    ws.carg[slot] = ca;
    ws.cbad[slot] = cb;
    __threadfence();  // partials visible device-wide before the counter moves
    const uint32_t prev = atomicAdd(&ws.count[row], 1u);
    s_last = (prev == (uint32_t)(nch - 1));
  }
  __syncthreads();
  if (!s_last) return;
  // ---- last workgroup of this row: merge the chunk partials in chunk order ----
  if (wid != 0) return;
  __threadfence();  // acquire: every chunk's partials are visible past this point
  float m_all = -INFINITY;
  int a_all = 0x7fffffff;
  int b_all = 0;
  for (int c = lane; c < nch; c += 64) {
    const float mc = ws.cmax[row * nch + c];
    const int ac = ws.carg[row * nch + c];
    b_all |= ws.cbad[row * nch + c];
    if (mc > m_all || (mc == m_all && ac < a_all)) {
      m_all = mc;
      a_all = ac;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m_all, o);
    const int oa = __shfl_xor(a_all, o);
    if (om > m_all || (om == m_all && oa < a_all)) {
      m_all = om;
      a_all = oa;
    }
  }
  b_all = wave_or_i(b_all);
  double z = 0.0;
  if (!greedy && m_all > -INFINITY) {
    // chunk order is fixed: lane c holds chunk c (plus c + 64, ...), then a fixed butterfly
    for (int c = lane; c < nch; c += 64) {
      const float mc = ws.cmax[row * nch + c];
      const double sc = ws.csum[row * nch + c];
      if (mc > -INFINITY) z += sc * exp(((double)mc - (double)m_all) * inv_t);
    }
    z = wave_sum_d(z);
  }
  if (lane == 0) {
    ws.count[row] = 0;  // leave the workspace ready for the next call
    const bool bad_row = b_all || !(m_all > -INFINITY);
    row_max[row] = bad_row ? NAN : m_all;
    if (row_sumexp) row_sumexp[row] = bad_row ? NAN : (float)z;
    if (row_argmax) row_argmax[row] = bad_row ? -1 : a_all;
    if (bad_row) report(status, SPEC_ERR_BAD_INPUT);
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

}  // namespace spectree

extern "C" size_t spec_tree_softmax_workspace_size(int64_t rows, int32_t vocab) {
  if (rows < 1 || vocab < 1) return 0;
  return spectree::sm_layout(rows, vocab, nullptr, nullptr);
}

extern "C" int spec_tree_softmax(const float* logits, int64_t rows, int32_t vocab, float temperature,
                                 float* row_max, float* row_sumexp, int32_t* row_argmax, float* probs,
                                 void* workspace, size_t workspace_bytes, int32_t* status, void* stream) {
  using namespace spectree;
  if (!logits || !row_max || rows < 1 || vocab < 1) return SPEC_ERR_INVALID_ARG;
  if (!(temperature >= 0.0f) || isinf(temperature)) return SPEC_ERR_INVALID_ARG;
  const bool greedy = temperature == 0.0f;
  if (!greedy && !row_sumexp) return SPEC_ERR_INVALID_ARG;
  if ((int64_t)sm_chunks(vocab) * rows > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  const size_t need = sm_layout(rows, vocab, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return SPEC_ERR_WORKSPACE;
  SmWorkspace ws;
  sm_layout(rows, vocab, (char*)workspace, &ws);
  const int nch = sm_chunks(vocab);
  const double inv_t = greedy ? 0.0 : 1.0 / (double)temperature;
  const ExpScale es = make_exp_scale(inv_t);
  const bool vec = (vocab % 4 == 0) && (((uintptr_t)logits & 15) == 0);
  dim3 grid((unsigned)(nch * rows));
  if (vec)
    hipLaunchKernelGGL(softmax_stats_kernel<true>, grid, dim3(kSmThreads), 0, (hipStream_t)stream, logits, vocab, nch,
                       inv_t, es, greedy ? 1 : 0, ws, row_max, row_sumexp, row_argmax, status);
  else
    hipLaunchKernelGGL(softmax_stats_kernel<false>, grid, dim3(kSmThreads), 0, (hipStream_t)stream, logits, vocab,
                       nch, inv_t, es, greedy ? 1 : 0, ws, row_max, row_sumexp, row_argmax, status);
  SPEC_LAUNCH_CHECK();
  if (probs && !greedy) {
    if (rows > 65535) return SPEC_ERR_UNSUPPORTED;
    dim3 g2((unsigned)((vocab + 255) / 256), (unsigned)rows);
    hipLaunchKernelGGL(softmax_probs_kernel, g2, dim3(256), 0, (hipStream_t)stream, logits, vocab, es, row_max,
                       row_sumexp, probs);
    SPEC_LAUNCH_CHECK();
  }
  return SPEC_OK;
}
