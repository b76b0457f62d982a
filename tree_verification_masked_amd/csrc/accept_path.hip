// Accepted path plus the bonus token.
//
// Tree-verification notes (zhangshuibai.github.io), "Tree Verification 详解" part C:
// the committed path runs from the root to the first rejection or a leaf and is
// unique; part G, step 6: the emitted tokens are the accepted ones followed by the
// bonus token.  One lane per request follows accepted_child (at most 63 steps).
// The rejection sampler can emit the same path from its own walk.
#include "common.hpp"

namespace spectree {

__global__ __launch_bounds__(256) void accept_path_kernel(const int32_t* __restrict__ accepted_child,
                                                          const int32_t* __restrict__ term_token,
                                                          const int32_t* __restrict__ tokens,
                                                          const int32_t* __restrict__ n_nodes, int32_t batch,
                                                          int32_t n_max, int32_t* __restrict__ path_nodes,
                                                          int32_t* __restrict__ out_tokens,
                                                          int32_t* __restrict__ accept_len, int32_t* status) {
  const int b = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (b >= batch) return;
  const int64_t base = (int64_t)b * n_max;
  bool bad;
  accept_len[b] = accept_walk(accepted_child + base, term_token + base, tokens + base, n_nodes[b], n_max,
                              path_nodes + base, out_tokens + base, &bad);
  if (bad) report(status, SPEC_ERR_BAD_INPUT);
}

}  // namespace spectree

extern "C" int spec_accept_path(const int32_t* accepted_child, const int32_t* term_token, const int32_t* tokens,
                                const int32_t* n_nodes, int32_t batch, int32_t n_max, int32_t* path_nodes,
                                int32_t* out_tokens, int32_t* accept_len, int32_t* status, void* stream) {
  if (!accepted_child || !term_token || !tokens || !n_nodes || !path_nodes || !out_tokens || !accept_len)
    return SPEC_ERR_INVALID_ARG;
  if (batch < 1 || n_max < 1 || n_max > 64) return SPEC_ERR_INVALID_ARG;
  dim3 grid((unsigned)((batch + 255) / 256));
  hipLaunchKernelGGL(spectree::accept_path_kernel, grid, dim3(256), 0, (hipStream_t)stream, accepted_child,
                     term_token, tokens, n_nodes, batch, n_max, path_nodes, out_tokens, accept_len, status);
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}
