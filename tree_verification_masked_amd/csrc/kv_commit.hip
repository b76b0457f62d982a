// KV commit and rollback after the accepted path.
//
// "EAGLE-4 Technical Deepdive" (blog.fal.ai), "EAGLE-4 verification trees and
// harness": after verification the accepted continuation is kept and the rejected
// KV-cache entries are freed.  Tree-verification notes (zhangshuibai.github.io),
// "Tree Verification 详解" part D.2: every tree node writes its own K/V, so the
// rejected nodes must leave the cache (rollback; paged caches free whole pages).
//
// Node j's K/V sits at logical position ctx + j.  The root stays at ctx; path node
// i (i = 1..L) moves from ctx + path[i] to ctx + i, and the committed length
// becomes ctx + 1 + L.  Since path[i] >= i, the destination of row i is never the
// source of a later row, so rows can be moved in increasing order in chunks; within
// a chunk every source is staged in LDS before any destination is written.  One
// workgroup per request moves all its KV heads (the accepted rows are few), then
// releases the pages that now hold only freed positions.
#include "common.hpp"

namespace spectree {

constexpr int kCommitLds = 65536;  // staging bytes per workgroup
constexpr int kCommitThreads = 256;
constexpr int kMaxFreed = 64;

struct CommitArgs {
  char *k, *v;
  int32_t elem;  // bytes per element
  int32_t* block_table;
  int32_t page_size, kv_capacity, n_pages;
  const int32_t *ctx_len, *n_nodes, *path_nodes, *accept_len;
  int32_t batch, n_max, hkv, head_dim;
  int32_t *new_len, *freed, *status;
};

// Byte offset of (request b, logical position t, KV head g); t and its page were
// validated by the caller of this helper.
__device__ inline int64_t commit_off(const CommitArgs& a, int b, int t, int g) {
  int64_t row;
  if (!a.block_table) {
    row = ((int64_t)b * a.kv_capacity + t) * a.hkv + g;
  } else {
    const int page = a.block_table[(int64_t)b * a.kv_capacity + t / a.page_size];
    row = ((int64_t)page * a.page_size + t % a.page_size) * a.hkv + g;
  }
  return row * a.head_dim * a.elem;
}

__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(CommitArgs a) {
  __shared__ __attribute__((aligned(16))) int4 s_buf[kCommitLds / 16];
  __shared__ int s_ok;
  const int tid = threadIdx.x, b = blockIdx.x;
  const int L = a.accept_len[b], n = a.n_nodes[b], ctx = a.ctx_len[b];
  const int32_t* path = a.path_nodes + (int64_t)b * a.n_max;
  if (a.freed)
    for (int j = tid; j < kMaxFreed; j += kCommitThreads) a.freed[(int64_t)b * kMaxFreed + j] = -1;
  if (tid == 0) {
    // the path must be a walk from the root inside the tree, and every position
    // of the tree must exist in the cache
    int ok = L >= 0 && n >= 1 && n <= a.n_max && L < n && ctx >= 0 && path[0] == 0;
    for (int i = 1; ok && i <= L; ++i) ok = path[i] > path[i - 1] && path[i] < n;
    if (ok) {
      const int64_t end = (int64_t)ctx + n;
      if (!a.block_table) {
        ok = end <= a.kv_capacity;
      } else {
        ok = end <= (int64_t)a.kv_capacity * a.page_size;
        for (int s = ctx / a.page_size; ok && s < (int)((end + a.page_size - 1) / a.page_size); ++s) {
          const int pg = a.block_table[(int64_t)b * a.kv_capacity + s];
          ok = pg >= 0 && pg < a.n_pages;
        }
      }
    }
    s_ok = ok;
    if (!ok) {
      a.new_len[b] = -1;
      if (L >= 0) report(a.status, SPEC_ERR_BAD_INPUT);  // (accept_len < 0: a request already refused)
    }
  }
  __syncthreads();
  if (!s_ok) return;
  const int pv = a.head_dim * a.elem / 16;       // 16-byte pieces per (position, head) vector
  const int per_row = a.hkv * 2 * pv;            // pieces per accepted row (K and V, every head)
  const int rows_per_chunk = kCommitLds / 16 / per_row;
  for (int i0 = 1; i0 <= L; i0 += rows_per_chunk) {
    const int nr = min(L - i0 + 1, rows_per_chunk);
    const int total = nr * per_row;
    for (int x = tid; x < total; x += kCommitThreads) {  // gather the chunk's sources
      const int r = x / per_row, y = x % per_row;
      const int g = y / (2 * pv), kv = (y / pv) & 1, p = y % pv;
      const char* base = kv ? a.v : a.k;
      s_buf[x] = *reinterpret_cast<const int4*>(base + commit_off(a, b, ctx + path[i0 + r], g) + p * 16);
    }
    __syncthreads();
    for (int x = tid; x < total; x += kCommitThreads) {  // then write its destinations
      const int r = x / per_row, y = x % per_row;
      const int g = y / (2 * pv), kv = (y / pv) & 1, p = y % pv;
      char* base = kv ? a.v : a.k;
      *reinterpret_cast<int4*>(base + commit_off(a, b, ctx + i0 + r, g) + p * 16) = s_buf[x];
    }
    __syncthreads();  // the buffer is reused and the next chunk's sources are read after these writes
  }
  if (tid == 0) {
    const int nl = ctx + 1 + L;
    a.new_len[b] = nl;
    if (a.block_table) {  // release the pages left holding only freed positions
      int32_t* tab = a.block_table + (int64_t)b * a.kv_capacity;
      const int first = (nl + a.page_size - 1) / a.page_size, end = (ctx + n + a.page_size - 1) / a.page_size;
      int j = 0;
      for (int s = first; s < end; ++s) {
        if (a.freed) a.freed[(int64_t)b * kMaxFreed + j] = tab[s];
        ++j;
        tab[s] = -1;
      }
    }
  }
}

}  // namespace spectree

extern "C" int spec_tree_kv_commit(void* k, void* v, int32_t dtype, int32_t* block_table, int32_t page_size,
                                   int32_t kv_capacity, int32_t n_pages, const int32_t* ctx_len,
                                   const int32_t* n_nodes, const int32_t* path_nodes, const int32_t* accept_len,
                                   int32_t batch, int32_t n_max, int32_t hkv, int32_t head_dim, int32_t* new_len,
                                   int32_t* freed_pages, int32_t* status, void* stream) {
  using namespace spectree;
  if (!k || !v || !ctx_len || !n_nodes || !path_nodes || !accept_len || !new_len) return SPEC_ERR_INVALID_ARG;
  if (batch < 1 || n_max < 1 || n_max > 64 || hkv < 1 || kv_capacity < 1) return SPEC_ERR_INVALID_ARG;
  if (block_table && (page_size < 1 || n_pages < 1)) return SPEC_ERR_INVALID_ARG;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return SPEC_ERR_UNSUPPORTED;
  const int elem = dtype == SPEC_F32 ? 4 : 2;
  if ((int64_t)hkv * head_dim * elem * 2 > kCommitLds) return SPEC_ERR_UNSUPPORTED;  // one row must fit the stage
  CommitArgs a;
  a.k = (char*)k;
  a.v = (char*)v;
  a.elem = elem;
  a.block_table = block_table;
  a.page_size = page_size;
  a.kv_capacity = kv_capacity;
  a.n_pages = n_pages;
  a.ctx_len = ctx_len;
  a.n_nodes = n_nodes;
  a.path_nodes = path_nodes;
  a.accept_len = accept_len;
  a.batch = batch;
  a.n_max = n_max;
  a.hkv = hkv;
  a.head_dim = head_dim;
  a.new_len = new_len;
  a.freed = freed_pages;
  a.status = status;
  hipLaunchKernelGGL(kv_commit_kernel, dim3((unsigned)batch), dim3(kCommitThreads), 0, (hipStream_t)stream, a);
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}
