// Ancestor mask of a flattened draft tree.
//
// Tree-verification notes (zhangshuibai.github.io), "Tree Verification 详解" part B:
// the tree is flattened breadth-first and every node may attend only to itself and
// its ancestors.  One wavefront handles one tree: lane i owns node i, validity is a
// wave vote and the ancestor sets come from pointer jumping over the parent links
// (tree_ancestors_wave, which the attention launch also uses when it is given the
// parent links), and every node sets its bit in its parent's child mask with one
// LDS atomic.
#include "common.hpp"

namespace spectree {

__global__ __launch_bounds__(256) void mask_build_kernel(const int32_t* __restrict__ parent,
                                                         const int32_t* __restrict__ n_nodes, int32_t batch,
                                                         int32_t n_max, uint64_t* __restrict__ anc_mask,
                                                         uint64_t* __restrict__ child_mask, int32_t* __restrict__ depth,
                                                         int32_t* status) {
  __shared__ unsigned long long s_kids[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int b = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  if (b >= batch) return;  // whole wavefront leaves together (no workgroup barrier below)
  s_kids[wv][lane] = 0;
  const int64_t base = (int64_t)b * n_max;
  const int n = n_nodes[b];
  const bool in_row = lane < n_max;
  const int p = in_row ? parent[base + lane] : -1;
  bool ok;
  const uint64_t a = tree_ancestors_wave(p, n, n_max, &ok);
  const bool node = lane < n;
  if (!ok) {
    if (in_row) {
      anc_mask[base + lane] = 0;
      child_mask[base + lane] = 0;
      depth[base + lane] = -1;
    }
    if (lane == 0) report(status, SPEC_ERR_BAD_TREE);
    return;
  }
  // the wavefront's own LDS row: in-order LDS operations of one wavefront need no barrier
  if (node && lane > 0) atomicOr(&s_kids[wv][p], 1ull << lane);
  __builtin_amdgcn_wave_barrier();
  const uint64_t kids = s_kids[wv][lane];
  if (in_row) {
    anc_mask[base + lane] = node ? a : 0ull;
    child_mask[base + lane] = node ? kids : 0ull;
    depth[base + lane] = node ? (__popcll(a) - 1) : -1;
  }
}

}  // namespace spectree

extern "C" int spec_tree_mask_build(const int32_t* parent, const int32_t* n_nodes, int32_t batch, int32_t n_max,
                                    uint64_t* anc_mask, uint64_t* child_mask, int32_t* depth, int32_t* status,
                                    void* stream) {
  if (!parent || !n_nodes || !anc_mask || !child_mask || !depth) return SPEC_ERR_INVALID_ARG;
  if (batch < 1 || n_max < 1 || n_max > 64) return SPEC_ERR_INVALID_ARG;
  const int trees_per_block = 4;
  dim3 grid((unsigned)((batch + trees_per_block - 1) / trees_per_block));
  hipLaunchKernelGGL(spectree::mask_build_kernel, grid, dim3(64 * trees_per_block), 0, (hipStream_t)stream, parent,
                     n_nodes, batch, n_max, anc_mask, child_mask, depth, status);
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}

extern "C" const char* spec_tree_version(void) { return "spectree 0.1 gfx950"; }
