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

// ---- wave64 reductions (fixed butterfly order, so results are deterministic) ----
__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline int wave_or_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o);
  return v;
}
__device__ inline uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl((uint32_t)v, src), hi = __shfl((uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}
// Inclusive prefix sum across the wave (Hillis-Steele, fixed order).
__device__ inline double wave_incl_scan_d(double v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    double t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
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

}  // namespace spectree

// ---- host side ----
#define SPEC_LAUNCH_CHECK()                                  \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP; \
  } while (0)
