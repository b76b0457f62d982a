/*
 * spec_tree.h -- C ABI of libspectree, the MI355X (gfx950) verification step of
 * EAGLE-style tree speculative decoding.
 *
 * One verification step over a flattened draft tree is:
 *   spec_tree_mask_build      parent links -> ancestor / child bitmasks, depths
 *   spec_tree_attention       tree-masked split-KV GQA attention
 *   spec_tree_softmax         per-node vocabulary softmax statistics (target, draft)
 *   spec_tree_reject_sample   lossless tree rejection sampling (or greedy at T = 0)
 *   spec_accept_path          longest accepted root-to-leaf path plus the bonus token
 *   spec_tree_verify_step     the whole step above in three launches (attention, logit
 *                             pass with the attention's split combine, sampler)
 *   spec_tree_kv_commit       keep the accepted path's K/V, free the rejected tree slots
 *   spec_tree_build_init      start EAGLE-2 draft trees at their roots
 *   spec_tree_expand          one EAGLE-2 expand round from the frontier's draft rows
 *   spec_tree_rerank          keep the top-N nodes by path value, flattened breadth-first
 *
 * Sources.  "EAGLE 演化史 (1 → 2 → 3) 与 DFlash 的回答" (zhangshuibai.github.io paper
 * notes), section "Tree Verification 详解": part B (BFS flattening and the
 * ancestor-only mask), part C (per-parent draft distribution, sibling fallthrough
 * on the residual, unique longest accepted path), part D.2 (cost split), part G
 * (worked example, bonus token at a leaf).  "Eagle vs DFlash: Best speculative
 * decoding methods" (gingerlabs.ai), section "Target-model decoding is serial"
 * (accept with probability min(1, p/q), resample from norm(max(0, p - q))).
 * "EAGLE-4 Technical Deepdive" (blog.fal.ai), "EAGLE-4 verification trees and
 * harness" (prefix + ancestors + self).  "The EAGLE Family: Speculating in Feature
 * Space" (consciousengines.com), "Why predict features instead of tokens?"
 * (next-token distribution = softmax of the LM-head output).
 *
 * Conventions shared by every entry point
 *  - Pointers named in the argument lists are DEVICE pointers unless stated, owned
 *    by the caller; arrays are row-major and contiguous.  The library never
 *    allocates or frees memory and never reads device memory from the host.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronises the host.  Results are valid once the stream
 *    reaches the call.
 *  - The return value reports what the host can check without touching device
 *    memory: SPEC_OK, or an error code below; on an error nothing is launched.
 *  - `status` (device int32, nullable) receives data errors found on the device:
 *    the first error code wins (atomic compare-and-swap from 0).  The caller zeroes
 *    it (with a kernel, not a memset, if the call is captured in a graph); the
 *    library never clears it.
 *  - Trees: node 0 is the root (the last committed token, never tested itself);
 *    nodes are flattened so that parent[i] < i (BFS order is one such order);
 *    parent[0] = -1; 1 <= n_nodes[b] <= n_max <= 64; entries i >= n_nodes[b] are
 *    padding and ignored.
 *  - Workspaces are caller-provided device buffers of at least the size the
 *    matching *_workspace_size query returns, zero-filled once before first use.
 *    Each call leaves its workspace zero-filled where that matters, so one buffer
 *    can be reused by consecutive calls of the same entry point on one stream.
 *    Calls that run concurrently need separate workspaces.
 *  - gfx950 only.  The library is stateless and reentrant across streams, except
 *    spec_tree_attention_noalloc, whose library-owned array is shared by every call
 *    on one GPU.
 */
#ifndef SPEC_TREE_H
#define SPEC_TREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPEC_OK = 0,
  SPEC_ERR_INVALID_ARG = -1, /* null pointer, size out of range, bad temperature  */
  SPEC_ERR_UNSUPPORTED = -2, /* a shape or dtype this build does not implement    */
  SPEC_ERR_BAD_TREE = -3,    /* device: parent[] does not describe a tree          */
  SPEC_ERR_BAD_INPUT = -4,   /* device: token or page id out of range, NaN/+inf    */
  SPEC_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required         */
  SPEC_ERR_HIP = -6,         /* a HIP launch failed                                */
  SPEC_ERR_TIMEOUT = -7      /* device: a bounded cross-workgroup wait gave up     */
} spec_status;

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* Markers written into the per-node sampling outputs. */
#define SPEC_NODE_NONE (-1)          /* no child accepted                          */
#define SPEC_NODE_NOT_EVALUATED (-2) /* node not visited by the walk               */
#define SPEC_NODE_BAD_REQUEST (-3)   /* request rejected (bad tree, token or row)  */

/*
 * Ancestor mask (tree notes, part B; fal.ai page, "verification trees").
 * For each request b and node i < n_nodes[b]:
 *   anc_mask[b,i]   bit j set iff node j is node i or one of its ancestors
 *   child_mask[b,p] bit i set iff parent[b,i] == p
 *   depth[b,i]      number of edges from the root (the caller's RoPE position of
 *                   node i is ctx_len[b] + depth[b,i])
 * parent, n_nodes: int32 [batch, n_max], [batch].  Outputs: uint64 [batch, n_max],
 * uint64 [batch, n_max], int32 [batch, n_max].  Padding entries get anc = child = 0
 * and depth = -1.  A request whose parent[] is not a tree gets all-zero masks,
 * depth -1 everywhere, and SPEC_ERR_BAD_TREE in status.
 * Host errors: batch < 1, n_max outside [1, 64], null pointers.
 */
int spec_tree_mask_build(const int32_t* parent, const int32_t* n_nodes, int32_t batch, int32_t n_max,
                         uint64_t* anc_mask, uint64_t* child_mask, int32_t* depth, int32_t* status, void* stream);

/*
 * Tree-masked attention (tree notes, parts B and D.2).  For request b, node
 * i < n_nodes[b] and query head h (KV head g = h / (hq / hkv)):
 *   visible keys = logical positions [0, ctx_len[b]) plus ctx_len[b] + j for
 *                  every node j that is node i or one of its ancestors
 * The ancestor sets come from exactly one of two inputs (the other is NULL):
 *   parent   int32 [batch, n_max]: the tree's parent links; the launch builds the
 *            ancestor sets itself (those spec_tree_mask_build would write), so no
 *            separate mask launch is needed.  A request whose links are not a tree
 *            rooted at node 0 (parent[b,0] = -1, 0 <= parent[b,i] < i) gets zero
 *            rows and SPEC_ERR_BAD_TREE.
 *   anc_mask uint64 [batch, n_max]: the ancestor rows, bit j of anc_mask[b,i] set
 *            when node j is visible to node i (as spec_tree_mask_build writes them).
 *   out[b,i,h,:] = softmax(scale * q . k) . v over the visible keys
 * The tree's own K/V rows sit at logical positions ctx_len[b] + j (node j), so the
 * caller writes them before this call.  Q and K carry RoPE already (node i at
 * position ctx_len[b] + depth[b,i]).
 *   q    [batch, n_max, hq, head_dim]           dtype
 *   k, v contiguous: [batch, kv_capacity, hkv, head_dim] (block_table == NULL)
 *        paged:      [n_pages, page_size, hkv, head_dim] with block_table int32
 *                    [batch, kv_capacity] listing the pages of each request in
 *                    logical order (kv_capacity = pages per request)
 *   out  [batch, n_max, hq, head_dim]           dtype; padding rows are zero
 * dtype SPEC_BF16 (fp32 accumulate) or SPEC_F32.  head_dim 64 or 128.
 * Query rows per KV head G = n_max * hq / hkv: bf16 with G >= 16 runs on MFMA
 * tiles, otherwise on a shuffle dot-product kernel.
 * max_kv_len bounds ctx_len[b] + n_nodes[b] over the batch; it sizes the key
 * splits (and the workspace), so a tight bound gives the best split.
 * Device errors: ctx_len[b] + n_nodes[b] beyond max_kv_len or the cache ->
 * SPEC_ERR_BAD_INPUT and the request's rows are written as zeros; a page id
 * outside [0, n_pages) -> SPEC_ERR_BAD_INPUT and the request's outputs are
 * unspecified (page 0 is read in its place, so no memory outside the pool is
 * touched).  A node whose ancestor mask lacks its own bit (the all-zero masks
 * spec_tree_mask_build writes for a bad tree) gets a zero row.
 * Host errors: null pointers, both or neither of parent and anc_mask, hq % hkv != 0, n_max outside [1, 64], page_size < 1
 * with a block table, scale not finite and positive, workspace too small;
 * SPEC_ERR_UNSUPPORTED for head_dim not 64/128, another dtype, or a block table
 * with pages of fewer than 16 tokens on the MFMA path (bf16, G >= 16).
 */
size_t spec_tree_attention_workspace_size(int32_t batch, int32_t n_max, int32_t hq, int32_t hkv, int32_t head_dim,
                                          int32_t max_kv_len);
int spec_tree_attention(const void* q, const void* k, const void* v, int32_t dtype, const int32_t* block_table,
                        int32_t page_size, int32_t kv_capacity, int32_t n_pages, const int32_t* ctx_len,
                        const int32_t* n_nodes, const int32_t* parent, const uint64_t* anc_mask, int32_t batch,
                        int32_t n_max, int32_t hq, int32_t hkv, int32_t head_dim, int32_t max_kv_len, float scale,
                        void* out, void* workspace, size_t workspace_bytes, int32_t* status, void* stream);

/*
 * spec_tree_attention for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, results and errors as spec_tree_attention, without the workspace: the
 * split partials go to a library-owned device array of
 * SPEC_TREE_ATTENTION_SCRATCH_BYTES per GPU (its address is resolved on the first
 * call on each device and kept; the array lives until the process ends).  Nothing
 * is allocated or freed by the call.  The array needs no clearing: every partial is
 * written before it is read.
 * Returns SPEC_ERR_WORKSPACE when the split partials of these sizes would exceed
 * the array (spec_tree_attention_workspace_size is an upper bound of what they
 * need), SPEC_ERR_HIP when the array's device address cannot be resolved.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (concurrent streams) race and must be serialised by the caller.
 */
#define SPEC_TREE_ATTENTION_SCRATCH_BYTES (16u << 20)
int spec_tree_attention_noalloc(const void* q, const void* k, const void* v, int32_t dtype,
                                const int32_t* block_table, int32_t page_size, int32_t kv_capacity, int32_t n_pages,
                                const int32_t* ctx_len, const int32_t* n_nodes, const int32_t* parent,
                                const uint64_t* anc_mask, int32_t batch, int32_t n_max, int32_t hq, int32_t hkv,
                                int32_t head_dim, int32_t max_kv_len, float scale, void* out, int32_t* status,
                                void* stream);

/*
 * Per-row vocabulary softmax statistics at temperature T ("The EAGLE Family",
 * "Why predict features instead of tokens?"; tree notes, parts A and D.2).
 *   row_max[r]    = max_x logits[r,x]
 *   row_sumexp[r] = sum_x exp((logits[r,x] - row_max[r]) / T)      (T > 0)
 *   row_argmax[r] = smallest x with logits[r,x] == row_max[r]       (nullable)
 *   probs[r,x]    = exp((logits[r,x] - row_max[r]) / T) / row_sumexp (nullable,
 *                   T > 0; meant for tests)
 *   chunk_max[r,c], chunk_sum[r,c] (nullable, both or neither): for chunk c of
 *                   spec_tree_softmax_chunk() tokens, the chunk's maximum m_c (NaN
 *                   if the chunk holds NaN or +inf) and
 *                   sum_x exp((logits[r,x] - m_c) / T) in fp64 -- the rejection
 *                   sampler merges its rows from them and draws bonus tokens at
 *                   leaves without another pass over the row.
 *                   [rows, ceil(vocab / chunk)].
 * logits: fp32 [rows, vocab].  -inf logits are probability 0.  A row holding NaN
 * or +inf, or only -inf, gets row_max = NaN and SPEC_ERR_BAD_INPUT in status.
 * T == 0 computes row_max and row_argmax only.
 * Host errors: rows < 1, vocab < 1, T < 0 or NaN, null outputs, workspace.
 */
int32_t spec_tree_softmax_chunk(void);
size_t spec_tree_softmax_workspace_size(int64_t rows, int32_t vocab);
int spec_tree_softmax(const float* logits, int64_t rows, int32_t vocab, float temperature, float* row_max,
                      float* row_sumexp, int32_t* row_argmax, float* probs, float* chunk_max, double* chunk_sum,
                      void* workspace, size_t workspace_bytes, int32_t* status, void* stream);

/*
 * The same statistics for the target rows (temperature T) and the draft rows
 * (temperature T_d) of a step in one launch, so the two vocabulary passes share
 * the GPU instead of running back to back.  Both arrays are fp32 [rows, vocab];
 * T > 0 and T_d > 0.
 *   chunk partials  tgt_chunk_max / tgt_chunk_sum and dft_chunk_max / dft_chunk_sum
 *                   [rows, ceil(vocab / chunk)] as spec_tree_softmax defines them
 *                   (each pair both or neither); a chunk holding NaN or +inf gets
 *                   maximum NaN.  These are what spec_tree_reject_sample reads.
 *   row statistics  tgt_max, tgt_sumexp, dft_max, dft_sumexp (all four or none) and
 *                   tgt_argmax (nullable) as spec_tree_softmax defines them.  With
 *                   none, no row merge is launched and both chunk pairs are required
 *                   -- the single vocabulary pass of a verification step.
 *   the tree        parent [batch, n_max] and n_nodes [batch] (both or neither;
 *                   rows = batch * n_max node rows, 1 <= n_max <= 64, chunk partials
 *                   only).  Tree notes, parts C and G: a node's draft distribution
 *                   only tests its children and a leaf draws from its target row, so
 *                   the draft partials are computed only for the rows of nodes with
 *                   at least one child (parent[b, c] == n for some n < c < n_nodes[b]);
 *                   the other rows' draft partials are left as they were.  The target
 *                   rows are all computed.  spec_tree_reject_sample reads exactly the
 *                   draft rows this computes.
 * Host errors (beyond spec_tree_softmax's): a tree with row statistics, n_max outside
 * [1, 64] or rows not a multiple of it, only one of parent / n_nodes.
 * The workspace query also leaves room, at its end, for the per-request counters
 * spec_tree_verify_step uses at T = 0 (left at zero by every call).
 */
size_t spec_tree_softmax_pair_workspace_size(int64_t rows, int32_t vocab);
int spec_tree_softmax_pair(const float* tgt_logits, float temperature, const float* dft_logits,
                           float draft_temperature, int64_t rows, int32_t vocab, const int32_t* parent,
                           const int32_t* n_nodes, int32_t n_max, float* tgt_max, float* tgt_sumexp,
                           int32_t* tgt_argmax, float* tgt_chunk_max, double* tgt_chunk_sum, float* dft_max,
                           float* dft_sumexp, float* dft_chunk_max, double* dft_chunk_sum, void* workspace,
                           size_t workspace_bytes, int32_t* status, void* stream);

/*
 * Tree rejection sampling (gingerlabs page, "Target-model decoding is serial";
 * tree notes, parts C and G).  Walks each request from the root.  At node n the
 * children c (parent[c] == n) are tested in ascending index against the target
 * distribution p_n = softmax(tgt_logits[n] / T) and the draft distribution at the
 * parent q_n = softmax(dft_logits[n] / T_d): child c with token x is accepted when
 * u_accept[c] < r(x) / q_n(x), where r starts as p_n and after each rejected
 * sibling becomes norm(max(0, r - q_n)) (unchanged if that mass is zero).  The
 * walk continues at an accepted child.  If every child is rejected the terminal
 * token is drawn from r by inverse CDF with u_sample[n] (smallest token whose
 * running sum exceeds u * total); at a leaf it is drawn from p_n the same way.
 * q(x) == 0 gives ratio +inf when r(x) > 0, else 0.
 * T == 0 is greedy: the first child whose token equals the target argmax is
 * accepted, the terminal token is that argmax; it reads tgt_max and tgt_argmax
 * (spec_tree_softmax at T = 0; a NaN maximum marks an invalid row) and the draft
 * and chunk inputs, uniforms and workspace may be NULL.
 * T > 0 reads the chunk partials of both arrays (spec_tree_softmax_pair or
 * spec_tree_softmax, same chunking) and merges each row's statistics itself;
 * tgt_max and tgt_argmax are not read.  The draft row of a node without children
 * takes no part (its draft partials are not read and need not be valid), so
 * spec_tree_softmax_pair given the tree may skip them.
 * Inputs: tgt_logits, dft_logits fp32 [batch, n_max, vocab]; tokens, parent int32
 * [batch, n_max]; n_nodes int32 [batch]; u_accept, u_sample fp32 [batch, n_max] in
 * [0, 1).
 * Outputs int32 [batch, n_max]: accepted_child[b,n] = accepted child,
 * SPEC_NODE_NONE, or SPEC_NODE_NOT_EVALUATED for nodes off the walk;
 * term_token[b,n] = the terminal token of the last node of the walk, else
 * SPEC_NODE_NOT_EVALUATED.  A request with a bad tree, a token outside
 * [0, vocab), an invalid target row or an invalid draft row of a node with
 * children gets accepted_child[b,0] = SPEC_NODE_BAD_REQUEST and a device error
 * code.
 * path_nodes, out_tokens [batch, n_max] and accept_len [batch] (int32, all three
 * or none, NULL to skip): the accepted path, exactly as spec_accept_path would
 * derive it from accepted_child and term_token, written by the same walk.
 * T > 0 needs the workspace of spec_tree_reject_sample_workspace_size, zero-filled
 * once; every call leaves it ready for the next.  Its first 16 bytes are uint32
 * counters, cumulative over calls (the caller may zero them between calls): word 0
 * counts the exact W(c) levels summed (one per rejected sibling, over all nodes),
 * word 1 the cross-workgroup waits that gave up; words 2-3 are reserved (0).
 * One kernel at T > 0 (several launches only when the grid exceeds one dispatch):
 * one planner workgroup per node slot (row statistics merged
 * from the chunk partials, the tree's verdict, the node's children and the
 * first-child test; a leaf's bonus; the report of a node that needs no chain) and
 * one workgroup per 4096-token chunk of every node, which keeps its logits in
 * registers as exact fixed-point masses.  After each rejected sibling the chunks of
 * a node publish their exact sums for the new threshold and read each other's (a
 * bounded wait; the chunks of one node run on one XCD when they fit there), so every
 * chunk takes the same next step; the terminal draw scans one chunk; the request's
 * last reported node walks from the root.  A wait that gives up marks its node
 * failed: SPEC_ERR_TIMEOUT in status, the request reported as SPEC_NODE_BAD_REQUEST,
 * the call still ends normally (spec_tree_reject_sample_set_wait_limit).
 * Host errors: T < 0 or NaN, T > 0 with T_d <= 0, null required pointers, only
 * some of the path outputs, sizes, workspace; SPEC_ERR_UNSUPPORTED for a
 * vocabulary above 256 chunks.
 */
size_t spec_tree_reject_sample_workspace_size(int32_t batch, int32_t n_max, int32_t vocab);
int spec_tree_reject_sample(const float* tgt_logits, float temperature, const float* tgt_max,
                            const int32_t* tgt_argmax, const float* tgt_chunk_max, const double* tgt_chunk_sum,
                            const float* dft_logits, float draft_temperature, const float* dft_chunk_max,
                            const double* dft_chunk_sum, const int32_t* tokens, const int32_t* parent,
                            const int32_t* n_nodes, const float* u_accept, const float* u_sample, int32_t batch,
                            int32_t n_max, int32_t vocab, int32_t* accepted_child, int32_t* term_token,
                            int32_t* path_nodes, int32_t* out_tokens, int32_t* accept_len, void* workspace,
                            size_t workspace_bytes, int32_t* status, void* stream);

/*
 * Bound on the polls of each cross-workgroup wait of spec_tree_reject_sample at
 * T > 0 (process-wide; 0 restores the default of 2^22).  A wait that reaches it
 * gives up: the node's result is marked failed, status gets SPEC_ERR_TIMEOUT, the
 * request is reported as SPEC_NODE_BAD_REQUEST, and the call still ends normally
 * with its workspace ready for the next call.  For tests of that path; the default
 * is never reached while the workgroups of one node can run together.
 */
void spec_tree_reject_sample_set_wait_limit(uint32_t polls);

/*
 * Accepted path plus bonus token (tree notes, parts C and G; gingerlabs page, "A
 * useful performance model": the accepted length counts drafted tokens, the bonus
 * is emitted on top).  Follows accepted_child from node 0 until SPEC_NODE_NONE.
 *   path_nodes [batch, n_max]  root first, then the accepted nodes; -1 padded
 *   out_tokens [batch, n_max]  tokens of the accepted nodes, then the terminal
 *                              token of the last node; -1 padded
 *   accept_len [batch]         number of accepted nodes; -1 for a rejected request
 * Host errors: null pointers, batch < 1, n_max outside [1, 64].
 */
int spec_accept_path(const int32_t* accepted_child, const int32_t* term_token, const int32_t* tokens,
                     const int32_t* n_nodes, int32_t batch, int32_t n_max, int32_t* path_nodes, int32_t* out_tokens,
                     int32_t* accept_len, int32_t* status, void* stream);

/*
 * The whole verification step (tree notes, part D.2: the tree-masked target pass,
 * then the verification of part C over every node's row) in one call, with the
 * results of spec_tree_attention (given the parent links), spec_tree_softmax_pair
 * given the tree (T > 0; spec_tree_softmax with row statistics of the target rows
 * at T = 0) and spec_tree_reject_sample with the path outputs, made by the same
 * kernels bit for bit.  Three launches instead of four: the attention's split
 * combine (when its plan has more than one key split) runs as extra workgroups of
 * the logit pass's launch, after its chunks; at T = 0 the greedy walk of a request
 * runs in the row merge's launch, by the wave that merges the request's last row.
 * The attention output is therefore complete only once the whole call has run.
 * Fields of SpecTreeStepArgs (every pointer a device pointer; sizes and layouts
 * those of the separate entry points):
 *   tree      parent, tokens [batch, n_max], n_nodes [batch]
 *   attention q, k, v, dtype, block_table, page_size, kv_capacity, n_pages,
 *             ctx_len, hq, hkv, head_dim, max_kv_len, scale, attn_out, and its
 *             workspace (spec_tree_attention_workspace_size)
 *   logits    tgt_logits, dft_logits (T > 0) [batch, n_max, vocab]; temperature,
 *             draft_temperature; T > 0: the chunk partials tgt_chunk_max,
 *             tgt_chunk_sum, dft_chunk_max, dft_chunk_sum [batch * n_max, nch];
 *             T = 0: tgt_max, tgt_sumexp, tgt_argmax [batch * n_max]; the logit
 *             workspace (spec_tree_softmax_pair_workspace_size of batch * n_max rows)
 *   sampling  u_accept, u_sample (T > 0); accepted_child, term_token, path_nodes,
 *             out_tokens [batch, n_max], accept_len [batch]; the sampler workspace
 *             (spec_tree_reject_sample_workspace_size, T > 0)
 *   status    as for every entry point
 * Host errors: a null `args`, and those of the three calls; at T = 0 every check of
 * the walk comes first (a workspace smaller than the query gives SPEC_ERR_WORKSPACE),
 * otherwise they are checked call by call, so an error of the logit pass or the
 * sampler can return after the attention was launched: then its combine has been
 * launched on its own, and the attention output is complete, but the sampling outputs
 * are not written.
 */
typedef struct SpecTreeStepArgs {
  const int32_t* parent;
  const int32_t* tokens;
  const int32_t* n_nodes;
  int32_t batch, n_max;
  const void* q;
  const void* k;
  const void* v;
  int32_t dtype;
  const int32_t* block_table;
  int32_t page_size, kv_capacity, n_pages;
  const int32_t* ctx_len;
  int32_t hq, hkv, head_dim, max_kv_len;
  float scale;
  void* attn_out;
  void* attn_workspace;
  size_t attn_workspace_bytes;
  const float* tgt_logits;
  const float* dft_logits;
  int32_t vocab;
  float temperature, draft_temperature;
  float* tgt_chunk_max;
  double* tgt_chunk_sum;
  float* dft_chunk_max;
  double* dft_chunk_sum;
  float* tgt_max;
  float* tgt_sumexp;
  int32_t* tgt_argmax;
  void* softmax_workspace;
  size_t softmax_workspace_bytes;
  const float* u_accept;
  const float* u_sample;
  int32_t* accepted_child;
  int32_t* term_token;
  int32_t* path_nodes;
  int32_t* out_tokens;
  int32_t* accept_len;
  void* sample_workspace;
  size_t sample_workspace_bytes;
  int32_t* status;
} SpecTreeStepArgs;
int spec_tree_verify_step(const SpecTreeStepArgs* args, void* stream);
/* sizeof(SpecTreeStepArgs) as the library was compiled (a binding's layout check). */
size_t spec_tree_step_args_size(void);

/*
 * KV commit and rollback after the path (fal.ai page, "EAGLE-4 verification trees
 * and harness": keep the accepted continuation, free the rejected KV entries; tree
 * notes, part D.2: rejected nodes must not stay in the cache).  Node j's K/V sits
 * at logical position ctx_len[b] + j; for path_nodes / accept_len as
 * spec_accept_path writes them, path node i (i = 1..L, L = accept_len[b]) is
 * moved from position ctx + path_nodes[b,i] to ctx + i for every KV head, K and V;
 * the root stays at ctx.  Sources are read before destinations are written, so
 * overlapping moves are exact.
 *   k, v          the cache of spec_tree_attention (contiguous or paged), in place
 *   n_layers      how many layers' caches to commit (>= 1): layer l's K and V start
 *                 at k + l * layer_stride and v + l * layer_stride elements; every
 *                 layer holds the tree at the same positions and shares block_table
 *   layer_stride  elements between consecutive layers (ignored for one layer; at
 *                 least one layer's size, batch * kv_capacity * hkv * head_dim or
 *                 n_pages * page_size * hkv * head_dim, so the layers never overlap)
 *   block_table   paged: pages whose slots hold only positions in
 *                 [new_len, ctx + n_nodes) are released: their entries become -1
 *   new_len [batch]      ctx + 1 + L, the committed length; -1 for a request that
 *                        was refused (accept_len < 0) or is invalid (path not an
 *                        increasing walk from the root inside the tree, a tree
 *                        position outside the cache, a bad page id), which is left
 *                        untouched (SPEC_ERR_BAD_INPUT in status for the invalid ones)
 *   freed_pages [batch, 64]  released page ids in slot order, -1 padded (nullable)
 * One workgroup per (request, layer), plus a per-request release kernel when
 * n_layers > 1; the moved bytes are n_layers * L * hkv * head_dim * elem * 2, read
 * and written once.
 * Host errors: null required pointers, batch < 1, n_max outside [1, 64], hkv < 1,
 * n_layers outside [1, 65535], a layer_stride below one layer's size, a block table
 * with page_size < 1 or n_pages < 1; SPEC_ERR_UNSUPPORTED for another
 * dtype, head_dim not 64/128, or hkv * head_dim * element size above 32 KiB.
 */
int spec_tree_kv_commit(void* k, void* v, int32_t dtype, int32_t n_layers, int64_t layer_stride,
                        int32_t* block_table, int32_t page_size,
                        int32_t kv_capacity, int32_t n_pages, const int32_t* ctx_len, const int32_t* n_nodes,
                        const int32_t* path_nodes, const int32_t* accept_len, int32_t batch, int32_t n_max,
                        int32_t hkv, int32_t head_dim, int32_t* new_len, int32_t* freed_pages, int32_t* status,
                        void* stream);

/*
 * Draft-tree construction, EAGLE-2 style (tree notes, part E.2: a node's value is
 * the product of the draft confidences on its root path; expand rounds grow the
 * frontier nodes of largest value by their top-k draft tokens; the rerank keeps the
 * N nodes of largest value, a connected subtree since value never grows along a
 * path; EAGLE family page, "EAGLE-2: context-aware dynamic trees": the kept nodes
 * are flattened with a tree mask for verification).  The output of
 * spec_tree_rerank is the parent[] / tokens / n_nodes input of the verify step.
 *
 * State of the trees under construction, caller-owned device arrays ([batch, cap]
 * unless stated), indexed by node id (root = 0; children get consecutive ids as
 * they are created: expanded nodes in frontier order, each node's children in top-k
 * order):
 *   cand_parent int32    parent id (-1 for the root)
 *   cand_token int32     token
 *   cand_path uint64     breadth-first key: depth in bits 63..60, then for
 *                        d = 1..depth the node's ancestor at depth d's rank among
 *                        its siblings (top-k order) in bits (63 - 4d)..(60 - 4d)
 *   cand_value double    product of the confidences on the root path (root 1)
 *   cand_conf double     the node's own confidence (draft probability of its token)
 *   cand_count [batch]   nodes so far
 *   frontier [batch, max_frontier], frontier_count [batch]
 *                        the nodes the next expand round grows, in the order
 *                        its draft rows must be given (value desc, ties to the
 *                        lower id); frontier_count 0 = nothing to grow
 * Limits: cap <= 1024, max_frontier <= 16, top_k <= 16, depth <= 15.
 */
int spec_tree_build_init(const int32_t* root_token, int32_t batch, int32_t cap, int32_t max_frontier,
                         int32_t* cand_parent, int32_t* cand_token, uint64_t* cand_path, double* cand_value,
                         double* cand_conf, int32_t* cand_count, int32_t* frontier, int32_t* frontier_count,
                         void* stream);

/*
 * One expand round.  draft_logits [batch, max_frontier, vocab] fp32: row j of
 * request b is the drafter's logits at node frontier[b][j] (rows j >=
 * frontier_count[b] are not read).  Each such node gets as children its top_k
 * tokens by logit (ties to the lower token id), with confidence
 * c = softmax(row / T_d)[token] (fp32 exponentials summed in fp64; c itself in
 * fp64) and value = value(node) * c.  The new frontier is the select_k nodes of
 * largest value (ties to the lower id) among
 *   policy 0  this round's children (EAGLE-2, layer by layer), or
 *   policy 1  every node without children below depth 15 (the best-first heap of
 *             DDTree, tree notes part E.4: whatever its depth, the most valuable
 *             unexpanded node is grown next; select_k 1 is the one-pop heap).
 * One read of every row.
 * Device errors (SPEC_ERR_BAD_INPUT in status; the request's frontier_count becomes
 * 0 and nothing is appended): a row with NaN or +inf or only -inf, a frontier entry
 * that is not an existing node or sits at depth 15, frontier_count above
 * max_frontier, or more than cap nodes.
 * Host errors: null pointers; batch < 1; max_frontier outside [1, 16]; top_k
 * outside [1, 16]; select_k outside [1, max_frontier]; policy not 0 or 1; cap
 * outside [1, 1024];
 * vocab < top_k; T_d not finite and positive; SPEC_ERR_UNSUPPORTED for vocab above
 * 262144; SPEC_ERR_WORKSPACE for a workspace smaller than
 * spec_tree_expand_workspace_size(batch, max_frontier, vocab) (0 = bad sizes).
 */
size_t spec_tree_expand_workspace_size(int32_t batch, int32_t max_frontier, int32_t vocab);
int spec_tree_expand(const float* draft_logits, int32_t vocab, float T_d, int32_t batch, int32_t max_frontier,
                     int32_t top_k, int32_t select_k, int32_t policy, int32_t cap, int32_t* cand_parent,
                     int32_t* cand_token,
                     uint64_t* cand_path, double* cand_value, double* cand_conf, int32_t* cand_count,
                     int32_t* frontier, int32_t* frontier_count, void* workspace, size_t workspace_bytes,
                     int32_t* status, void* stream);

/*
 * Rerank and flatten.  Keeps the root and the n_final - 1 other nodes of largest
 * value (ties to the shallower node, then the lower id), in breadth-first order:
 * by depth, then the parent's flattened index, then sibling (top-k) order.
 *   parent, tokens, cand_id [batch, n_final]  flattened tree (parent[0] = -1;
 *                        parent[i] < i), its tokens, and each flattened node's id in
 *                        the state; entries i >= n_nodes[b] are -1
 *   n_nodes [batch]      min(n_final, cand_count[b])
 * Device errors: cand_count outside [1, cap] -> n_nodes 0 and SPEC_ERR_BAD_INPUT;
 * a kept node whose parent is not kept (a state that is not a tree) -> n_nodes 0
 * and SPEC_ERR_BAD_TREE.
 * Host errors: null pointers; batch < 1; cap outside [1, 1024]; n_final outside
 * [1, 64].
 */
int spec_tree_rerank(const int32_t* cand_parent, const int32_t* cand_token, const uint64_t* cand_path,
                     const double* cand_value, const int32_t* cand_count, int32_t batch, int32_t cap,
                     int32_t n_final, int32_t* parent, int32_t* tokens, int32_t* n_nodes, int32_t* cand_id,
                     int32_t* status, void* stream);

/* Library version string (static storage). */
const char* spec_tree_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_TREE_H */
