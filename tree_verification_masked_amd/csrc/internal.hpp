// Host-side calls shared between the library's translation units (not exported).
#pragma once

#include "attn_combine.hpp"
#include "greedy_walk.hpp"

namespace spectree {

// attention.hip: the attention launch; with `defer`, its split combine is described
// there instead of launched.
int attention_launch(const void* q, const void* k, const void* v, int32_t dtype, const int32_t* block_table,
                     int32_t page_size, int32_t kv_capacity, int32_t n_pages, const int32_t* ctx_len,
                     const int32_t* n_nodes, const int32_t* parent, const uint64_t* anc_mask, int32_t batch,
                     int32_t n_max, int32_t hq, int32_t hkv, int32_t head_dim, int32_t max_kv_len, float scale,
                     void* out, void* workspace, size_t workspace_bytes, int32_t* status, void* stream,
                     AttnCombine* defer);
int attention_combine_launch(const AttnCombine& c, void* stream);

// softmax.hip: spec_tree_softmax and spec_tree_softmax_pair, whose chunk launch also
// runs the rows of `comb` (when given, with rows > 0); softmax_call's row merge also
// runs the greedy walk of `walk` (when given: rows are batch * n_max node rows, and
// req_count holds batch zeroed counters, left at zero).
int softmax_call(const float* logits, int64_t rows, int32_t vocab, float temperature, float* row_max,
                 float* row_sumexp, int32_t* row_argmax, float* probs, float* chunk_max, double* chunk_sum,
                 void* workspace, size_t workspace_bytes, int32_t* status, void* stream, const AttnCombine* comb,
                 const GreedyArgs* walk, uint32_t* req_count);
// The offset of the step's per-request counters in a softmax_pair workspace.
size_t softmax_pair_counters_offset(int64_t rows, int32_t vocab);
int softmax_pair_call(const float* tgt_logits, float temperature, const float* dft_logits, float draft_temperature,
                      int64_t rows, int32_t vocab, const int32_t* parent, const int32_t* n_nodes, int32_t n_max,
                      float* tgt_max, float* tgt_sumexp, int32_t* tgt_argmax, float* tgt_chunk_max,
                      double* tgt_chunk_sum, float* dft_max, float* dft_sumexp, float* dft_chunk_max,
                      double* dft_chunk_sum, void* workspace, size_t workspace_bytes, int32_t* status, void* stream,
                      const AttnCombine* comb);

}  // namespace spectree
