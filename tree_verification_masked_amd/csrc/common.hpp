// Shared device and host helpers of libspectree (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "spec_tree.h"

namespace spectree {

constexpr int kWave = 64;
// Vocabulary chunk shared by the softmax statistics and the samplers: chunk c of a
// row covers tokens [c * kChunk, (c + 1) * kChunk).
constexpr int kChunk = 4096;

// First data error wins; later errors leave the word unchanged.
__device__ inline void report(int32_t* status, int32_t code) {
  if (status) atomicCAS(status, 0, code);
}

// ---- wave64 cross-lane steps through DPP ----
// Reductions use row-local permutes (quad swaps, half-row and row mirrors) and the
// two row broadcasts; the total ends in lane 63 and is read back as a scalar, so
// every lane sees it.  Scans use row shifts plus the row broadcasts.  Everything
// stays in the vector ALU (no LDS permute) and the order of operations is fixed,
// so results are deterministic.  Callers keep all 64 lanes active.
constexpr int kDppQuad1032 = 0xb1, kDppQuad2301 = 0x4e, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;

// DPP move of v; lanes of rows outside kRowMask (or with no source lane) get `old`.
template <int kCtrl, int kRowMask = 0xf>
__device__ inline int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, kCtrl, kRowMask, 0xf, false);
}
template <int kCtrl, int kRowMask = 0xf>
__device__ inline float dpp_f(float old, float v) {
  return __int_as_float(dpp_i<kCtrl, kRowMask>(__float_as_int(old), __float_as_int(v)));
}
template <int kCtrl, int kRowMask = 0xf>
__device__ inline long long dpp_ll(long long old, long long v) {
  const int lo = dpp_i<kCtrl, kRowMask>((int)(uint32_t)old, (int)(uint32_t)v);
  const int hi = dpp_i<kCtrl, kRowMask>((int)(uint32_t)((unsigned long long)old >> 32),
                                        (int)(uint32_t)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}
template <int kCtrl, int kRowMask = 0xf>
__device__ inline double dpp_d(double old, double v) {
  return __longlong_as_double(dpp_ll<kCtrl, kRowMask>(__double_as_longlong(old), __double_as_longlong(v)));
}
__device__ inline int lane63_i(int v) { return __builtin_amdgcn_readlane(v, 63); }
__device__ inline float lane63_f(float v) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63)); }
__device__ inline long long lane63_ll(long long v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((unsigned long long)v >> 32), 63);
  return (long long)(((unsigned long long)hi << 32) | lo);
}
__device__ inline double lane63_d(double v) { return __longlong_as_double(lane63_ll(__double_as_longlong(v))); }

__device__ inline float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<kDppQuad1032>(v, v));
  v = fmaxf(v, dpp_f<kDppQuad2301>(v, v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppBcast15, 0xa>(v, v));
  v = fmaxf(v, dpp_f<kDppBcast31, 0xc>(v, v));
  return lane63_f(v);
}
__device__ inline float wave_sum_f(float v) {
  v += dpp_f<kDppQuad1032>(0.0f, v);
  v += dpp_f<kDppQuad2301>(0.0f, v);
  v += dpp_f<kDppHalfMirror>(0.0f, v);
  v += dpp_f<kDppMirror>(0.0f, v);
  v += dpp_f<kDppBcast15, 0xa>(0.0f, v);
  v += dpp_f<kDppBcast31, 0xc>(0.0f, v);
  return lane63_f(v);
}
__device__ inline double wave_sum_d(double v) {
  v += dpp_d<kDppQuad1032>(0.0, v);
  v += dpp_d<kDppQuad2301>(0.0, v);
  v += dpp_d<kDppHalfMirror>(0.0, v);
  v += dpp_d<kDppMirror>(0.0, v);
  v += dpp_d<kDppBcast15, 0xa>(0.0, v);
  v += dpp_d<kDppBcast31, 0xc>(0.0, v);
  return lane63_d(v);
}
__device__ inline long long wave_sum_ll(long long v) {
  v += dpp_ll<kDppQuad1032>(0, v);
  v += dpp_ll<kDppQuad2301>(0, v);
  v += dpp_ll<kDppHalfMirror>(0, v);
  v += dpp_ll<kDppMirror>(0, v);
  v += dpp_ll<kDppBcast15, 0xa>(0, v);
  v += dpp_ll<kDppBcast31, 0xc>(0, v);
  return lane63_ll(v);
}
__device__ inline int wave_max_i(int v) {
  v = max(v, dpp_i<kDppQuad1032>(v, v));
  v = max(v, dpp_i<kDppQuad2301>(v, v));
  v = max(v, dpp_i<kDppHalfMirror>(v, v));
  v = max(v, dpp_i<kDppMirror>(v, v));
  v = max(v, dpp_i<kDppBcast15, 0xa>(v, v));
  v = max(v, dpp_i<kDppBcast31, 0xc>(v, v));
  return lane63_i(v);
}
__device__ inline int wave_or_i(int v) {
  v |= dpp_i<kDppQuad1032>(0, v);
  v |= dpp_i<kDppQuad2301>(0, v);
  v |= dpp_i<kDppHalfMirror>(0, v);
  v |= dpp_i<kDppMirror>(0, v);
  v |= dpp_i<kDppBcast15, 0xa>(0, v);
  v |= dpp_i<kDppBcast31, 0xc>(0, v);
  return lane63_i(v);
}
// Inclusive prefix sums across the wave in lane order (lanes without a source in a
// shift add 0).
__device__ inline int wave_incl_scan_i(int v) {
  v += dpp_i<kDppShr1>(0, v);
  v += dpp_i<kDppShr2>(0, v);
  v += dpp_i<kDppShr4>(0, v);
  v += dpp_i<kDppShr8>(0, v);
  v += dpp_i<kDppBcast15, 0xa>(0, v);
  v += dpp_i<kDppBcast31, 0xc>(0, v);
  return v;
}
__device__ inline long long wave_incl_scan_ll(long long v) {
  v += dpp_ll<kDppShr1>(0, v);
  v += dpp_ll<kDppShr2>(0, v);
  v += dpp_ll<kDppShr4>(0, v);
  v += dpp_ll<kDppShr8>(0, v);
  v += dpp_ll<kDppBcast15, 0xa>(0, v);
  v += dpp_ll<kDppBcast31, 0xc>(0, v);
  return v;
}
__device__ inline double wave_incl_scan_d(double v, int /*lane*/) {
  v += dpp_d<kDppShr1>(0.0, v);
  v += dpp_d<kDppShr2>(0.0, v);
  v += dpp_d<kDppShr4>(0.0, v);
  v += dpp_d<kDppShr8>(0.0, v);
  v += dpp_d<kDppBcast15, 0xa>(0.0, v);
  v += dpp_d<kDppBcast31, 0xc>(0.0, v);
  return v;
}
__device__ inline uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl((uint32_t)v, src), hi = __shfl((uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// Ancestor set of a flattened draft tree, one wavefront per tree ("Tree Verification
// 详解" part B: a node sees itself and its ancestors).  Lane i passes node i's parent
// link p (-1 past n_max) and gets the bitmask of node i and its ancestors (0 for
// lanes at or past n).  *ok: n lies in [1, n_max] and the links form a tree rooted
// at node 0 with every parent ahead of its child (wave-uniform).  The sets come
// from pointer jumping: six doubling steps cover depth 63.
__device__ inline uint64_t tree_ancestors_wave(int p, int n, int n_max, bool* ok) {
  const int lane = threadIdx.x & 63;
  const bool n_ok = n >= 1 && n <= n_max;
  const bool node = n_ok && lane < n;
  const bool link_ok = !node || (lane == 0 ? p == -1 : (p >= 0 && p < lane));
  *ok = n_ok && __all(link_ok);
  if (!*ok) return 0ull;
  // a: ancestors at distance < 2^t (self included); jp: the ancestor at distance 2^t
  uint64_t a = node ? (1ull << lane) : 0ull;
  int jp = node ? p : -1;
#pragma unroll
  for (int t = 0; t < 6; ++t) {
    const int src = jp < 0 ? lane : jp;
    const uint64_t a_src = shfl_u64(a, src);
    const int jp_src = __shfl(jp, src);
    if (jp >= 0) {
      a |= a_src;
      jp = jp_src;
    }
  }
  return a;
}

// exp(d / T) for d <= 0 written as 2^(d * log2(e) / T); the scale is carried as an
// fp32 pair (hi + lo) so that its rounding does not bias every element the same way.
struct ExpScale {
  float hi, lo;
};
inline ExpScale make_exp_scale(double inv_t) {
  double s = 1.4426950408889634 * inv_t;
  ExpScale e;
  e.hi = (float)s;
  e.lo = (float)(s - (double)e.hi);
  return e;
}
// d = -inf (a masked logit) is clamped to the most negative finite float first, so
// that d * lo can never be +inf and meet -inf inside the fma.
__device__ inline float exp_scaled(float d, ExpScale s) {
  d = fmaxf(d, -3.402823466e38f);
  return __builtin_amdgcn_exp2f(fmaf(d, s.hi, d * s.lo));
}

__device__ inline bool is_bad_logit(float x) { return isnan(x) || x == INFINITY; }

// ---- publishing small results across workgroups (last-block merges) ----
// Values meant for another workgroup are written with agent-scope atomic stores
// (they bypass the non-coherent caches), the writer waits for its stores to
// complete before bumping the counter, and the reader uses agent-scope atomic
// loads.  This keeps the merge free of whole-L2 write-back / invalidate fences.
template <typename T>
__device__ inline void pub_store(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ inline T pub_load(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// All of this thread's prior stores have completed (compiler fences keep the
// surrounding memory operations on their side of the wait).
__device__ inline void stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Returns the counter value before the increment.
__device__ inline uint32_t pub_arrive(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Accepted path of one request from its per-node results, by one thread (tree
// notes, parts C and G: the path runs from the root to the first node without an
// accepted child and is unique; the emitted tokens are the accepted ones followed
// by that node's terminal token).  acc, term, tok: n_max entries of the request
// (LDS or global).  pn, ot receive n_max entries: -1 padding, then the path.
// Returns the number of accepted nodes; -1 for a request marked invalid (or with
// n outside [1, n_max]), and -1 with *bad set when the results are inconsistent.
__device__ inline int accept_walk(const int32_t* acc, const int32_t* term, const int32_t* tok, int n, int n_max,
                                  int32_t* pn, int32_t* ot, bool* bad) {
  *bad = false;
  for (int i = 0; i < n_max; ++i) pn[i] = ot[i] = -1;
  if (n < 1 || n > n_max || acc[0] == SPEC_NODE_BAD_REQUEST) return -1;
  int cur = 0, len = 0;
  bool ok = true;
  pn[0] = 0;
  for (int step = 0; step < n_max; ++step) {
    const int nxt = acc[cur];
    if (nxt < 0) break;
    if (nxt <= cur || nxt >= n || len + 1 >= n_max) {
      ok = false;
      break;
    }
    cur = nxt;
    ++len;
    pn[len] = cur;
    ot[len - 1] = tok[cur];
  }
  if (ok && (acc[cur] != SPEC_NODE_NONE || term[cur] < 0)) ok = false;
  if (!ok) {
    for (int i = 0; i < n_max; ++i) pn[i] = ot[i] = -1;
    *bad = true;
    return -1;
  }
  ot[len] = term[cur];
  return len;
}

}  // namespace spectree

// ---- host side ----
#define SPEC_LAUNCH_CHECK()                                  \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP; \
  } while (0)
