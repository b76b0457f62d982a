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
// workgroup per (request, layer) moves all the layer's KV heads (the accepted rows
// are few); every layer's cache holds the tree at the same positions and shares the
// page table.  Pages that now hold only freed positions are released once per
// request, after every layer has read its sources: by the same workgroup when there
// is one layer, else by a second, per-request kernel on the same stream.
#include "common.hpp"

namespace spectree {

constexpr int kCommitLds = 65536;  // staging bytes per workgroup
constexpr int kCommitThreads = 256;
constexpr int kMaxFreed = 64;

struct CommitArgs {
  char *k, *v;
  int64_t layer_bytes;  // distance between consecutive layers' caches
  int32_t elem;         // bytes per element
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

// Whether request b's commit is valid (one wavefront, every lane gets the answer):
// the path must be a walk from the root inside the tree, and every position of the
// tree must exist in the cache.  Lane i checks path entry i (L < n <= 64) and the
// i-th page slot of the tree's span (at most 64 slots: n <= 64 positions).
__device__ inline bool commit_valid(const CommitArgs& a, int b, int lane) {
  const int L = a.accept_len[b], n = a.n_nodes[b], ctx = a.ctx_len[b];
  const int32_t* path = a.path_nodes + (int64_t)b * a.n_max;
  const bool head = L >= 0 && n >= 1 && n <= a.n_max && L < n && ctx >= 0;
  if (!head) return false;
  bool ok = true;
  if (lane <= L) {
    const int p = path[lane];
    ok = lane == 0 ? p == 0 : (p > path[lane - 1] && p < n);
  }
  const int64_t end = (int64_t)ctx + n;
  if (!a.block_table) {
    ok = ok && end <= a.kv_capacity;
  } else {
    ok = ok && end <= (int64_t)a.kv_capacity * a.page_size;
    const int s = ctx / a.page_size + lane;
    if (ok && s < (int)((end + a.page_size - 1) / a.page_size)) {
      const int pg = a.block_table[(int64_t)b * a.kv_capacity + s];
      ok = pg >= 0 && pg < a.n_pages;
    }
  }
  return __all(ok) != 0;
}

// The per-request end of a commit (one wavefront): new length, error report, page
// release (lane i releases the i-th freed slot).  Runs only after every layer of the
// request has read its sources.
__device__ inline void commit_finish(const CommitArgs& a, int b, bool ok, int lane) {
  const int L = a.accept_len[b], n = a.n_nodes[b], ctx = a.ctx_len[b];
  if (!ok) {
    if (lane == 0) {
      a.new_len[b] = -1;
      if (L >= 0) report(a.status, SPEC_ERR_BAD_INPUT);  // (accept_len < 0: a request already refused)
    }
    return;
  }
  const int nl = ctx + 1 + L;
  if (lane == 0) a.new_len[b] = nl;
  if (a.block_table) {  // release the pages left holding only freed positions
    int32_t* tab = a.block_table + (int64_t)b * a.kv_capacity;
    const int first = (nl + a.page_size - 1) / a.page_size, end = (ctx + n + a.page_size - 1) / a.page_size;
    const int s = first + lane;
    if (s < end) {
      if (a.freed) a.freed[(int64_t)b * kMaxFreed + lane] = tab[s];
      tab[s] = -1;
    }
  }
}

// grid (batch, layers).  FINISH: one layer, so the same workgroup ends the request.
template <bool FINISH>
__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(CommitArgs a) {
  __shared__ __attribute__((aligned(16))) int4 s_buf[kCommitLds / 16];
  __shared__ int s_ok;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, b = blockIdx.x;
  const int L = a.accept_len[b], ctx = a.ctx_len[b];
  const int32_t* path = a.path_nodes + (int64_t)b * a.n_max;
  if (wid == 0) {
    if (FINISH && a.freed) a.freed[(int64_t)b * kMaxFreed + lane] = -1;
    const bool ok = commit_valid(a, b, lane);
    if (lane == 0) s_ok = ok;
    if (FINISH && !ok) commit_finish(a, b, false, lane);
  }
  __syncthreads();
  if (!s_ok) return;
  char* const lk = a.k + (int64_t)blockIdx.y * a.layer_bytes;
  char* const lv = a.v + (int64_t)blockIdx.y * a.layer_bytes;
  const int pv = a.head_dim * a.elem / 16;       // 16-byte pieces per (position, head) vector
  const int per_row = a.hkv * 2 * pv;            // pieces per accepted row (K and V, every head)
  const int rows_per_chunk = kCommitLds / 16 / per_row;
  for (int i0 = 1; i0 <= L; i0 += rows_per_chunk) {
    const int nr = min(L - i0 + 1, rows_per_chunk);
    const int total = nr * per_row;
    for (int x = tid; x < total; x += kCommitThreads) {  // gather the chunk's sources
      const int r = x / per_row, y = x % per_row;
      const int g = y / (2 * pv), kv = (y / pv) & 1, p = y % pv;
      const char* base = kv ? lv : lk;
      s_buf[x] = *reinterpret_cast<const int4*>(base + commit_off(a, b, ctx + path[i0 + r], g) + p * 16);
    }
    __syncthreads();
    for (int x = tid; x < total; x += kCommitThreads) {  // then write its destinations
      const int r = x / per_row, y = x % per_row;
      const int g = y / (2 * pv), kv = (y / pv) & 1, p = y % pv;
      char* base = kv ? lv : lk;
      *reinterpret_cast<int4*>(base + commit_off(a, b, ctx + i0 + r, g) + p * 16) = s_buf[x];
    }
    __syncthreads();  // the buffer is reused and the next chunk's sources are read after these writes
  }
  if (FINISH && wid == 0) commit_finish(a, b, true, lane);
}

// After the moves of every layer: one wavefront per request.
__global__ __launch_bounds__(64) void kv_commit_finish_kernel(CommitArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  if (a.freed) a.freed[(int64_t)b * kMaxFreed + lane] = -1;
  commit_finish(a, b, commit_valid(a, b, lane), lane);
}

}  // namespace spectree

extern "C" int spec_tree_kv_commit(void* k, void* v, int32_t dtype, int32_t n_layers, int64_t layer_stride,
                                   int32_t* block_table, int32_t page_size,
                                   int32_t kv_capacity, int32_t n_pages, const int32_t* ctx_len,
                                   const int32_t* n_nodes, const int32_t* path_nodes, const int32_t* accept_len,
                                   int32_t batch, int32_t n_max, int32_t hkv, int32_t head_dim, int32_t* new_len,
                                   int32_t* freed_pages, int32_t* status, void* stream) {
  using namespace spectree;
  if (!k || !v || !ctx_len || !n_nodes || !path_nodes || !accept_len || !new_len) return SPEC_ERR_INVALID_ARG;
  if (batch < 1 || n_max < 1 || n_max > 64 || hkv < 1 || kv_capacity < 1) return SPEC_ERR_INVALID_ARG;
  if (n_layers < 1 || n_layers > 65535) return SPEC_ERR_INVALID_ARG;
  if (block_table && (page_size < 1 || n_pages < 1)) return SPEC_ERR_INVALID_ARG;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return SPEC_ERR_UNSUPPORTED;
  const int elem = dtype == SPEC_F32 ? 4 : 2;
  if ((int64_t)hkv * head_dim * elem * 2 > kCommitLds) return SPEC_ERR_UNSUPPORTED;  // one row must fit the stage
  if (n_layers > 1) {  // the layers' caches must not overlap
    const int64_t layer_elems = block_table ? (int64_t)n_pages * page_size * hkv * head_dim
                                            : (int64_t)batch * kv_capacity * hkv * head_dim;
    if (layer_stride < layer_elems) return SPEC_ERR_INVALID_ARG;
  }
  CommitArgs a;
  a.k = (char*)k;
  a.v = (char*)v;
  a.layer_bytes = n_layers > 1 ? layer_stride * elem : 0;
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
  if (n_layers == 1) {
    hipLaunchKernelGGL(kv_commit_kernel<true>, dim3((unsigned)batch), dim3(kCommitThreads), 0, (hipStream_t)stream,
                       a);
    SPEC_LAUNCH_CHECK();
    return SPEC_OK;
  }
  hipLaunchKernelGGL(kv_commit_kernel<false>, dim3((unsigned)batch, (unsigned)n_layers), dim3(kCommitThreads), 0,
                     (hipStream_t)stream, a);
  SPEC_LAUNCH_CHECK();
  hipLaunchKernelGGL(kv_commit_finish_kernel, dim3((unsigned)batch), dim3(64), 0, (hipStream_t)stream, a);
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}
